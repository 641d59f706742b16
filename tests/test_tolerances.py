"""CPU checks of the comparison helpers the GPU parity tests use (no GPU)."""
import numpy as np
import torch

from gpu_common import TOL_GEMV, bf16_storage_excess, half_ulp_bf16, rel_err_per_vector


def _rne_bf16(x: np.ndarray) -> np.ndarray:
    # torch's CPU cast: round to nearest even
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def test_half_ulp_bf16_closed_forms():
    v = np.array([1.0, 1.5, 2.0, -3.0, 0.75, 0.0, 2.0 ** -130])
    # bf16 keeps 8 significand bits: spacing 2^(e - 7), half of it 2^(e - 8)
    assert np.array_equal(half_ulp_bf16(v), [2.0 ** -8, 2.0 ** -8, 2.0 ** -7, 2.0 ** -7, 2.0 ** -9, 0.0, 2.0 ** -138])
    # one RNE cast never moves a value by more than the allowance
    x = np.random.default_rng(1).standard_normal(100_000) * 10.0 ** np.random.default_rng(2).integers(-3, 4, 100_000)
    r = _rne_bf16(x.astype(np.float32)).astype(np.float64)
    x32 = x.astype(np.float32).astype(np.float64)
    assert np.all(np.abs(r - x32) <= half_ulp_bf16(np.maximum(np.abs(r), np.abs(x32))))


def test_storage_excess_passes_casts_and_fails_real_errors():
    rng = np.random.default_rng(3)
    ref = rng.standard_normal((50, 37))
    # a float32 result within 1e-6 of ref, cast once: within the bar
    h = _rne_bf16((ref * (1 + rng.standard_normal(ref.shape) * 1e-6)).astype(np.float32))
    assert np.all(bf16_storage_excess(h, ref) <= 0.0)
    # the check is one-sided: excess <= ||float32 error|| / ||ref|| always
    # (the cast adds at most the allowance), so an excess above the bar proves
    # the float32 result is off by more; errors below bf16's own step are not
    # visible in a bf16 output.  A 1 % error is caught.
    bad = _rne_bf16((ref * (1 + rng.choice([-1.0, 1.0], ref.shape) * 1e-2)).astype(np.float32))
    assert np.all(bf16_storage_excess(bad, ref) > TOL_GEMV)
    # the plain per-vector relative error is the ratio of norms
    y = np.array([[3.0, 4.0]])
    assert np.allclose(rel_err_per_vector(y + [[0.0, 5e-3]], y), [1e-3])
