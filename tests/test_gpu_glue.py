"""GPU parity of the MoE-layer glue entry points against the oracle.

iqk_moe_gemv_swiglu: h = silu(gate . x) * (up . x) stored as bf16; bar: the
matvec's 1e-3 per vector on top of the bf16 cast's exact allowance of half a
bf16 spacing per element (``gpu_common.bf16_storage_excess``).  iqk_moe_gemv_combine:
y[t] = sum_j w[t, j] W_j x_j in float32; bar: |y - ref| <= 1e-3 *
sum_j |w_j| ||W_j x_j|| per token (the combine may cancel, so the bound is
taken on the parts)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import dequant_iqk_moe_amd as q
from gpu_common import TOL_GEMV, announce, bf16_round, bf16_storage_excess, to_dev

pytestmark = pytest.mark.gpu

KS, K, R4 = 1, 2, 3


def _weights(fmt, E, out, n, seed):
    wire = synth.wire(fmt, E * out, n, seed)
    return q.Weights.from_wire(fmt, E, out, n, wire), oracle.pack(fmt, wire, E * out, n)


def _inputs(seed, T, k, E, x_slots, n):
    ids = synth.topk_ids(T, k, E, seed + 3)
    x = bf16_round(synth.normal((T, x_slots, n), seed + 4))
    return ids, x


@pytest.mark.parametrize("fmt", [KS, K, R4])
@pytest.mark.parametrize("n,I,T,k,E,x_slots", [
    (4096, 64, 3, 6, 16, 1),
    (2048, 36, 2, 4, 8, 4),     # ragged: 36 rows in units of 2 gate + 2 up rows
    (512, 20, 5, 3, 6, 1),      # 8-row units: 4 gate + 4 up rows per wave iteration
    (4096, 2048, 1, 6, 12, 1),  # the gate/up geometry, fewer experts
])
def test_swiglu_parity(fmt, n, I, T, k, E, x_slots):
    seed = 700 + fmt + n // 256 + I
    announce(f"swiglu fmt={fmt} n={n} I={I} T={T} k={k} E={E} slots={x_slots}")
    w, s = _weights(fmt, E, 2 * I, n, seed)
    values, grid = synth.values_table(seed + 1), synth.ternary_grid(seed + 2)
    ids, x = _inputs(seed, T, k, E, x_slots, n)
    h = q.moe_gemv_swiglu(w, to_dev(x, torch.bfloat16), to_dev(ids), values, to_dev(grid), x_slots=x_slots)
    h = h.float().cpu().numpy()
    ref = oracle.swiglu(oracle.moe(fmt, s, E, 2 * I, n, x, ids, values, grid, x_slots=x_slots))
    assert h.shape == (T, k, I)
    err = bf16_storage_excess(h, ref)
    assert np.all(err <= TOL_GEMV), err.max()


@pytest.mark.parametrize("fmt", [KS, K, R4])
@pytest.mark.parametrize("n,out,T,k,E,x_slots", [
    (2048, 72, 3, 6, 8, 6),
    (4096, 40, 5, 4, 10, 1),    # shared input: sum_j w_j W_j x
    (512, 24, 7, 8, 12, 8),     # k = 8, the most slots
    (2048, 4100, 1, 6, 8, 6),   # ragged tail, one token over many blocks
    (2048, 16, 40, 6, 9, 6),    # many tokens, few rows: one block per token
])
def test_combine_parity(fmt, n, out, T, k, E, x_slots):
    seed = 800 + fmt + n // 256 + out
    announce(f"combine fmt={fmt} n={n} out={out} T={T} k={k} E={E} slots={x_slots}")
    w, s = _weights(fmt, E, out, n, seed)
    values, grid = synth.values_table(seed + 1), synth.ternary_grid(seed + 2)
    ids, x = _inputs(seed, T, k, E, x_slots, n)
    rw = np.random.default_rng(seed + 5).dirichlet(np.ones(k), size=T).astype(np.float32)
    y = q.moe_gemv_combine(w, to_dev(x, torch.bfloat16), to_dev(ids), to_dev(rw), values, to_dev(grid),
                           x_slots=x_slots).cpu().numpy()
    parts = oracle.moe(fmt, s, E, out, n, x, ids, values, grid, x_slots=x_slots)
    ref = oracle.combine(parts, rw)
    scale = np.sum(np.abs(rw)[:, :, None] * np.linalg.norm(parts, axis=-1, keepdims=True), axis=1)[:, 0]
    err = np.linalg.norm(y - ref, axis=-1) / scale
    assert np.all(err <= TOL_GEMV), err.max()


def test_combine_deterministic_and_invalid_ids():
    fmt, n, out, E, T, k = K, 2048, 64, 10, 6, 6
    w, s = _weights(fmt, E, out, n, 900)
    values = synth.values_table(901)
    ids, x = _inputs(900, T, k, E, k, n)
    rw = np.random.default_rng(905).dirichlet(np.ones(k), size=T).astype(np.float32)
    xd, rwd = to_dev(x, torch.bfloat16), to_dev(rw)
    announce("combine determinism / invalid ids")
    a = q.moe_gemv_combine(w, xd, to_dev(ids), rwd, values).cpu().numpy()
    b = q.moe_gemv_combine(w, xd, to_dev(ids), rwd, values).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    bad = ids.copy()
    bad[2, 4] = -1
    bad[4, 0] = E
    c = q.moe_gemv_combine(w, xd, to_dev(bad), rwd, values).cpu().numpy()
    assert np.all(np.isnan(c[[2, 4]]))
    keep = [0, 1, 3, 5]
    assert np.array_equal(c[keep].view(np.uint32), a[keep].view(np.uint32))


def test_swiglu_invalid_ids_give_nan_rows():
    fmt, n, I, E = KS, 2048, 48, 5
    w, s = _weights(fmt, E, 2 * I, n, 910)
    values = synth.values_table(911)
    ids = np.array([[0, 7, -1, 2]], np.int32)
    x = bf16_round(synth.normal((1, 1, n), 912))
    announce("swiglu invalid ids")
    h = q.moe_gemv_swiglu(w, to_dev(x, torch.bfloat16), to_dev(ids), values).float().cpu().numpy()
    assert np.all(np.isnan(h[0, 1])) and np.all(np.isnan(h[0, 2]))
    ref = oracle.swiglu(oracle.moe(fmt, s, E, 2 * I, n, x, ids, values))
    assert np.all(bf16_storage_excess(h[0, [0, 3]], ref[0, [0, 3]]) <= TOL_GEMV)


# ---------------------------------------------------------------------------
# standalone glue kernels (the prefill paths' layer steps)
# ---------------------------------------------------------------------------

def test_standalone_swiglu_matches_oracle_and_the_epilogue():
    """iqk_swiglu on a gate/up output: oracle bar on random inputs (including
    large |g| where exp overflows), and bit-identical to the decode epilogue
    on the same projection"""
    rng = np.random.default_rng(1000)
    P, I = 37, 52
    y = (rng.standard_normal((P, 2 * I)) * 4).astype(np.float32)
    y[0, :4] = [0.0, -0.0, 95.0, -95.0]   # silu(0) = 0; exp(-g) overflow and underflow
    announce("standalone swiglu")
    h = q.swiglu(to_dev(y)).float().cpu().numpy()
    ref = oracle.swiglu(y.astype(np.float64))
    assert np.all(bf16_storage_excess(h, ref) <= TOL_GEMV)
    # against the epilogue: the same gate/up sums through either route
    fmt, n, I2, E, T, k = K, 2048, 64, 8, 3, 6
    w, s = _weights(fmt, E, 2 * I2, n, 1001)
    values = synth.values_table(1002)
    ids, x = _inputs(1001, T, k, E, 1, n)
    xd, idd = to_dev(x, torch.bfloat16), to_dev(ids)
    h_epi = q.moe_gemv_swiglu(w, xd, idd, values)
    h_two = q.swiglu(q.moe_gemv(w, xd, idd, values))
    assert np.array_equal(h_epi.cpu().view(torch.int16).numpy(), h_two.cpu().view(torch.int16).numpy())


def test_standalone_combine_matches_oracle_and_the_epilogue():
    rng = np.random.default_rng(1010)
    T, k, out = 9, 6, 40
    y = rng.standard_normal((T, k, out)).astype(np.float32)
    rw = rng.dirichlet(np.ones(k), size=T).astype(np.float32)
    y[3, 2, 5] = np.nan
    announce("standalone combine")
    yc = q.combine(to_dev(y), to_dev(rw)).cpu().numpy()
    ref = oracle.combine(y.astype(np.float64), rw)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(yc), nan) and nan.sum() == 1 and nan[3, 5]
    scale = np.sum(np.abs(rw)[:, :, None] * np.abs(y), axis=1)
    assert np.all(np.abs(yc[~nan] - ref[~nan]) <= 1e-6 * scale[~nan])
    # against the epilogue: the same per-slot sums through either route
    fmt, n, out2, E, T2 = KS, 2048, 48, 10, 4
    w, s = _weights(fmt, E, out2, n, 1011)
    values = synth.values_table(1012)
    ids, x = _inputs(1011, T2, k, E, k, n)
    rw2 = rng.dirichlet(np.ones(k), size=T2).astype(np.float32)
    xd, idd, rwd = to_dev(x, torch.bfloat16), to_dev(ids), to_dev(rw2)
    y_epi = q.moe_gemv_combine(w, xd, idd, rwd, values).cpu().numpy()
    parts = q.moe_gemv(w, xd, idd, values, x_slots=k)
    y_two = q.combine(parts, rwd).cpu().numpy()
    pv = parts.cpu().numpy()
    scale = np.sum(np.abs(rw2)[:, :, None] * np.abs(pv), axis=1)
    assert np.all(np.abs(y_epi - y_two) <= 1e-6 * scale)
