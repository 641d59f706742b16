"""Pins for the oracle's routed-expert product and routing gather.

"mlx-iqk" package description, "Surface" section: ``proj(x, indices)`` is the
switch-linear interface -- one output vector per (token, slot) pair, the
weights of the selected expert applied to the token's activation -- and a
sorted prefill reads each expert once.

Pins: the product reduces to numpy's float64 matmul of the dequantized
weights; a one-hot activation returns one weight column exactly; the
routing gather equals numpy's stable argsort; structural invariants
(duplicated tokens give equal rows, per-slot inputs select their own slot).
"""
import numpy as np
import pytest

import oracle
import synth

KS, K, R4 = oracle.IQ2_KS, oracle.IQ2_K, oracle.IQ1_S_R4


def _case(fmt, E, out, n, seed):
    w = synth.wire(fmt, E * out, n, seed)
    s = oracle.pack(fmt, w, E * out, n)
    return s, synth.values_table(seed + 1), synth.ternary_grid(seed + 2)


@pytest.mark.parametrize("fmt", [KS, K, R4])
def test_moe_reduces_to_float64_matmul(fmt):
    E, out, n, T, k = 5, 12, 512, 3, 2
    s, values, grid = _case(fmt, E, out, n, 50 + fmt)
    W = oracle.dequant(fmt, s, E * out, n, values, grid).reshape(E, out, n).astype(np.float64)
    x = synth.normal((T, n), 60)
    ids = synth.topk_ids(T, k, E, 61)
    y = oracle.moe(fmt, s, E, out, n, x, ids, values, grid)
    for t in range(T):
        for j in range(k):
            ref = W[ids[t, j]] @ x[t].astype(np.float64)
            np.testing.assert_allclose(y[t, j], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("fmt", [KS, K, R4])
def test_one_hot_activation_returns_a_weight_column(fmt):
    E, out, n = 3, 8, 256
    s, values, grid = _case(fmt, E, out, n, 70 + fmt)
    W = oracle.dequant(fmt, s, E * out, n, values, grid).reshape(E, out, n)
    for kk in (0, 31, 32, 255):
        x = np.zeros((1, n), np.float32)
        x[0, kk] = 1.0
        y = oracle.moe(fmt, s, E, out, n, x, np.array([[2, 0]], np.int32), values, grid)
        assert np.array_equal(y[0, 0], W[2, :, kk].astype(np.float64))
        assert np.array_equal(y[0, 1], W[0, :, kk].astype(np.float64))


def test_per_slot_inputs_and_duplicate_tokens():
    fmt, E, out, n = K, 4, 8, 256
    s, values, _ = _case(fmt, E, out, n, 80)
    x = synth.normal((2, 3, n), 81)
    x[1] = x[0]
    ids = np.array([[0, 3, 1], [0, 3, 1]], np.int32)
    y = oracle.moe(fmt, s, E, out, n, x, ids, values, None, x_slots=3)
    assert np.array_equal(y[0], y[1])
    W = oracle.dequant(fmt, s, E * out, n, values).reshape(E, out, n).astype(np.float64)
    np.testing.assert_allclose(y[0, 2], W[1] @ x[0, 2].astype(np.float64), rtol=1e-12)


def test_invalid_expert_id_gives_nan_row():
    fmt, E, out, n = KS, 2, 4, 256
    s, values, _ = _case(fmt, E, out, n, 90)
    y = oracle.moe(fmt, s, E, out, n, synth.normal((1, n), 1), np.array([[1, 7]], np.int32), values)
    assert np.all(np.isfinite(y[0, 0])) and np.all(np.isnan(y[0, 1]))


def test_bf16_weight_variant_rounds_each_weight():
    fmt, E, out, n = KS, 2, 6, 256
    s, values, _ = _case(fmt, E, out, n, 95)
    x = synth.normal((1, n), 96)
    Wb = oracle.dequant(fmt, s, E * out, n, values, None, oracle.BF16).reshape(E, out, n)
    Wb = (Wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y = oracle.moe(fmt, s, E, out, n, x, np.array([[1]], np.int32), values, w_bf16=True)
    np.testing.assert_allclose(y[0, 0], Wb[1] @ x[0].astype(np.float64), rtol=1e-12)


@pytest.mark.parametrize("T,k,E", [(1, 6, 256), (8, 6, 256), (512, 6, 256), (37, 3, 5), (0, 6, 16)])
def test_route_is_a_stable_expert_sort(T, k, E):
    ids = synth.topk_ids(T, k, E, 100 + T) if T else np.zeros((0, k), np.int32)
    counts, offsets, perm, bad = oracle.route(ids, E)
    flat = ids.ravel()
    assert bad == 0
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))


def test_route_skips_invalid_ids():
    ids = np.array([3, -1, 0, 9, 3, 1], np.int32)
    counts, offsets, perm, bad = oracle.route(ids, 4)
    assert bad == 2
    assert list(counts) == [1, 1, 0, 2]
    assert list(perm) == [2, 5, 0, 4]
