"""GPU parity of the grouped decode matvec (one decode pass per selected
expert, shared by all of its pairs) against the oracle.

Bar: rel. err <= 1e-3 per output vector against the float32-weight product
(the same fixed-point activation and integer sums as the per-pair matvec).
The per-pair matvec forms each pair's sums in the same order, so the two
also agree to float32 rounding (1e-6 per vector)."""
import numpy as np
import pytest
import torch

import oracle
import synth
import dequant_iqk_moe_amd as q
from gpu_common import TOL_GEMV, announce, bf16_round, rel_err_per_vector, to_dev

pytestmark = pytest.mark.gpu

KS, K, R4 = 1, 2, 3
TOL_SAME_SUMS = 1e-6


def _weights(fmt, E, out, n, seed):
    wire = synth.wire(fmt, E * out, n, seed)
    return q.Weights.from_wire(fmt, E, out, n, wire), oracle.pack(fmt, wire, E * out, n)


@pytest.mark.parametrize("x_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("fmt", [KS, K, R4])
@pytest.mark.parametrize("n,out,T,k,E,x_slots", [
    (4096, 72, 12, 4, 8, 1),     # ~6 pairs per expert, ragged last row group
    (2048, 72, 9, 4, 6, 4),      # per-pair input (down)
    (512, 72, 20, 3, 5, 1),      # ~12 per expert: three or four passes
    (2048, 4100, 3, 2, 3, 1),    # many groups per expert, ragged tail
    (512, 8, 300, 6, 40, 6),     # 45 pairs per expert, two-row groups
    (4096, 520, 40, 6, 64, 1),   # more row groups than one workgroup: runs span experts
])
def test_grouped_parity(fmt, n, out, T, k, E, x_slots, x_dtype):
    seed = 1300 + fmt + n // 256 + out + T
    announce(f"grouped gemv fmt={fmt} n={n} out={out} T={T} k={k} E={E} slots={x_slots} x={x_dtype}")
    w, s = _weights(fmt, E, out, n, seed)
    values, grid = synth.values_table(seed + 1), synth.ternary_grid(seed + 2)
    x = synth.normal((T, x_slots, n), seed + 3)
    if x_dtype == torch.bfloat16:
        x = bf16_round(x)
    ids = synth.topk_ids(T, k, E, seed + 4)
    xd, idd, gd = to_dev(x, x_dtype), to_dev(ids), to_dev(grid)
    y = q.moe_gemv_grouped(w, xd, idd, values, gd, x_slots=x_slots).cpu().numpy()
    ref = oracle.moe(fmt, s, E, out, n, x, ids, values, grid, x_slots=x_slots)
    err = rel_err_per_vector(y, ref)
    assert np.all(err <= TOL_GEMV), err.max()
    y1 = q.moe_gemv(w, xd, idd, values, gd, x_slots=x_slots).cpu().numpy()
    assert np.all(rel_err_per_vector(y, y1.astype(np.float64)) <= TOL_SAME_SUMS)


def test_grouped_invalid_ids_nan_and_deterministic():
    fmt, n, out, E, T, k = K, 2048, 40, 6, 25, 4
    w, s = _weights(fmt, E, out, n, 1400)
    values = synth.values_table(1401)
    x = bf16_round(synth.normal((T, 1, n), 1402))
    ids = synth.topk_ids(T, k, E, 1403)
    ids[2, 1] = -1
    ids[9, 3] = E
    announce("grouped gemv: invalid ids, determinism, skewed routing")
    xd, idd = to_dev(x, torch.bfloat16), to_dev(ids)
    sentinel = torch.full((T, k, out), 5.0, dtype=torch.float32, device="cuda")
    y = q.moe_gemv_grouped(w, xd, idd, values, y=sentinel).cpu().numpy()
    assert np.all(np.isnan(y[2, 1])) and np.all(np.isnan(y[9, 3]))  # NaN rows, as on the per-pair path
    valid = (ids >= 0) & (ids < E)
    ref = oracle.moe(fmt, s, E, out, n, x, np.where(valid, ids, 0), values)
    assert np.all(rel_err_per_vector(y[valid], ref[valid]) <= TOL_GEMV)
    y2 = q.moe_gemv_grouped(w, xd, idd, values, y=sentinel.clone()).cpu().numpy()
    assert np.array_equal(y.view(np.uint32), y2.view(np.uint32))


@pytest.mark.parametrize("fmt", [KS, R4])
def test_grouped_skewed_routing(fmt):
    """one expert holds most pairs (many passes of a few tokens) while
    others hold one or none"""
    n, out, E, T, k = 4096, 256, 12, 60, 2
    seed = 1500 + fmt
    w, s = _weights(fmt, E, out, n, seed)
    values, grid = synth.values_table(seed + 1), synth.ternary_grid(seed + 2)
    x = bf16_round(synth.normal((T, 1, n), seed + 3))
    ids = synth.topk_ids(T, k, E, seed + 4)
    ids[:50, 0] = 3
    ids[:50, 1] = np.where(ids[:50, 1] == 3, 4, ids[:50, 1])
    announce(f"grouped gemv skewed fmt={fmt}")
    y = q.moe_gemv_grouped(w, to_dev(x, torch.bfloat16), to_dev(ids), values, to_dev(grid)).cpu().numpy()
    ref = oracle.moe(fmt, s, E, out, n, x, ids, values, grid)
    assert np.all(rel_err_per_vector(y, ref) <= TOL_GEMV)


@pytest.mark.parametrize("T,expect", [(2, "gemv"), (6, "gemv"), (7, "grouped_gemv"), (8, "grouped_gemv"),
                                      (12, "grouped_gemv"), (13, "fused_prefill"), (20, "fused_prefill")])
def test_auto_dispatch_by_pairs_per_expert(T, expect):
    """in = 4096, 16 experts, 2 slots: pairs per expert T/8 up to 3/4 (T = 6)
    pick the per-pair matvec, up to 3/2 (T = 12) the grouped matvec, beyond
    the fused prefill; each result meets its path's bar"""
    fmt, n, out, E, k = K, 4096, 64, 16, 2
    seed = 1600 + T
    w, s = _weights(fmt, E, out, n, seed)
    values = synth.values_table(seed + 1)
    x = bf16_round(synth.normal((T, 1, n), seed + 3))
    ids = synth.topk_ids(T, k, E, seed + 4)
    announce(f"auto dispatch T={T}")
    y, path = q.moe_auto(w, to_dev(x, torch.bfloat16), to_dev(ids), values)
    assert path == expect
    ref = oracle.moe(fmt, s, E, out, n, x, ids, values)
    tol = TOL_GEMV if path != "fused_prefill" else 2e-2
    assert np.all(rel_err_per_vector(y.cpu().numpy(), ref) <= tol)
    # a float32 activation never takes the prefill
    y32, path32 = q.moe_auto(w, to_dev(x, torch.float32), to_dev(ids), values)
    assert path32 == ("gemv" if expect == "gemv" else "grouped_gemv")
    assert np.all(rel_err_per_vector(y32.cpu().numpy(), ref) <= TOL_GEMV)



def test_auto_dispatch_narrow_input():
    """in = 2048: per-pair matvec up to 3/4 pair per expert, then the fused prefill"""
    fmt, n, out, E, k = KS, 2048, 48, 16, 2
    w, s = _weights(fmt, E, out, n, 1700)
    values = synth.values_table(1701)
    for T, expect in ((6, "gemv"), (8, "fused_prefill")):
        x = bf16_round(synth.normal((T, 1, n), 1702 + T))
        ids = synth.topk_ids(T, k, E, 1710 + T)
        announce(f"auto dispatch narrow T={T}")
        y, path = q.moe_auto(w, to_dev(x, torch.bfloat16), to_dev(ids), values)
        assert path == expect
        ref = oracle.moe(fmt, s, E, out, n, x, ids, values)
        tol = TOL_GEMV if path == "gemv" else 2e-2
        assert np.all(rel_err_per_vector(y.cpu().numpy(), ref) <= tol)



@pytest.mark.parametrize("fmt", [K, R4])
def test_grouped_many_experts(fmt):
    """1500 experts: the plan scans them in two chunks"""
    n, out, E, T, k = 512, 16, 1500, 300, 6
    seed = 1900 + fmt
    announce(f"grouped gemv many experts fmt={fmt}")
    w, s = _weights(fmt, E, out, n, seed)
    values, grid = synth.values_table(seed + 1), synth.ternary_grid(seed + 2)
    x = bf16_round(synth.normal((T, 1, n), seed + 3))
    ids = synth.topk_ids(T, k, E, seed + 4)
    y = q.moe_gemv_grouped(w, to_dev(x, torch.bfloat16), to_dev(ids), values, to_dev(grid)).cpu().numpy()
    ref = oracle.moe(fmt, s, E, out, n, x, ids, values, grid)
    assert np.all(rel_err_per_vector(y, ref) <= TOL_GEMV)
