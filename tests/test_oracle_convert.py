"""Pins for the oracle's IEEE conversions against library routines.

The reconstruction reads an fp16 scale (the "mlx-iqk" description's "Format"
section: dv is an fp16 row / super-block scale) and the dequantizer's f16 /
bf16 outputs are one round-to-nearest-even cast of the float32 result.  Here
the oracle's hand-written conversions are checked against numpy's float16
casts and torch's CPU bfloat16 cast, both IEEE round-to-nearest-even.
"""
import numpy as np
import pytest
import torch

import oracle


def _specials():
    bits = np.array([
        0x00000000, 0x80000000, 0x00000001, 0x80000001, 0x007FFFFF, 0x00800000,
        0x7F7FFFFF, 0xFF7FFFFF, 0x7F800000, 0xFF800000, 0x3F800000, 0xBF800000,
        0x33800000, 0x33000000, 0x33000001, 0x387FC000, 0x38800000, 0x477FE000,
        0x477FEFFF, 0x477FF000, 0x477FF001, 0x47800000, 0x3F808000, 0x3F818000,
        0x3F807FFF, 0x3F808001, 0x7F7F8000, 0x7F7F7FFF,
    ], np.uint32)
    return bits.view(np.float32)


def test_f16_to_f32_all_halves_match_numpy():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_to_f32_array(h)
    ref = h.view(np.float16).astype(np.float32)
    finite = ~np.isnan(ref)
    assert np.array_equal(got[finite].view(np.uint32), ref[finite].view(np.uint32))
    assert np.all(np.isnan(got[~finite]))
    # NaN payloads survive: quiet bit and upper payload bits are kept
    assert np.array_equal(got[~finite].view(np.uint32) >> 13 & 0x3FF, h[~finite].astype(np.uint32) & 0x3FF)


def _random_f32(count, seed):
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2**32, size=count, dtype=np.uint64).astype(np.uint32)
    # concentrate half the sample around the fp16 range (exponents 100..160)
    e = rng.integers(100, 161, size=count // 2).astype(np.uint32)
    bits[: count // 2] = (bits[: count // 2] & 0x807FFFFF) | (e << 23)
    return bits.view(np.float32)


def test_f32_to_f16_matches_numpy_rne():
    x = np.concatenate([_specials(), _random_f32(400_000, 11)])
    got = oracle.f32_to_f16_array(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    finite = ~np.isnan(x)
    assert np.array_equal(got[finite], ref[finite])
    assert np.all(np.isnan(got[~finite].view(np.float16)))


def test_f32_to_bf16_matches_torch_rne():
    x = np.concatenate([_specials(), _random_f32(400_000, 12)])
    got = oracle.f32_to_bf16_array(x)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    finite = ~np.isnan(x)
    assert np.array_equal(got[finite], ref[finite])
    nan_out = (got[~finite].astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isnan(nan_out))


def test_rne_ties_by_hand():
    # bf16: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0);
    # 1 + 3*2^-8 is a tie between 1+2^-7 and 1+2^-6 -> even (1 + 2^-6)
    assert oracle.f32_to_bf16_bits(1.0 + 2.0**-8) == 0x3F80
    assert oracle.f32_to_bf16_bits(1.0 + 3 * 2.0**-8) == 0x3F82
    # f16: 65520 ties between 65504 and 65536 -> overflows to +inf
    assert oracle.f32_to_f16_bits(65520.0) == 0x7C00
    assert oracle.f32_to_f16_bits(65519.996) == 0x7BFF
    # f16 smallest subnormal is 2^-24; 2^-25 ties with 0 -> 0, a hair more -> 2^-24
    assert oracle.f32_to_f16_bits(2.0**-25) == 0x0000
    assert oracle.f32_to_f16_bits(np.nextafter(np.float32(2.0**-25), np.float32(1))) == 0x0001
    assert oracle.f16_to_f32(0x0001) == 2.0**-24
    assert oracle.f16_to_f32(0x03FF) == 1023 * 2.0**-24
    assert oracle.f16_to_f32(0x7BFF) == 65504.0


@pytest.mark.slow
def test_exhaustive_f32_casts():
    step = 1 << 24
    for start in range(0, 1 << 32, step):
        bits = np.arange(start, start + step, dtype=np.uint64).astype(np.uint32)
        x = bits.view(np.float32)
        finite = ~np.isnan(x)
        got16 = oracle.f32_to_f16_array(x)
        with np.errstate(over="ignore"):
            ref16 = x.astype(np.float16).view(np.uint16)
        assert np.array_equal(got16[finite], ref16[finite])
        gotb = oracle.f32_to_bf16_array(x)
        refb = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(gotb[finite], refb[finite])
