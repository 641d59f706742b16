"""GPU parity of the fused prefill (dequantization inside the MFMA grouped
GEMM) against the oracle.

The fused kernel multiplies with exactly the bf16 weights iqk_dequant
writes, so against the oracle's bf16-weight product (float64 sums of the
RNE-rounded weights times the bf16 activations) the only difference is the
float32 accumulation order: bar 1e-4 per output vector, which a single
mis-decoded weight breaks.  Against the float32-weight product the bf16 bar
2e-2 applies."""
import numpy as np
import pytest
import torch

import oracle
import synth
import dequant_iqk_moe_amd as q
from gpu_common import TOL_BF16, announce, bf16_round, rel_err_per_vector, to_dev

pytestmark = pytest.mark.gpu

KS, K, R4 = 1, 2, 3
TOL_SAME_WEIGHTS = 1e-4


def _weights(fmt, E, out, n, seed):
    wire = synth.wire(fmt, E * out, n, seed)
    return q.Weights.from_wire(fmt, E, out, n, wire), oracle.pack(fmt, wire, E * out, n)


@pytest.mark.parametrize("fmt", [KS, K, R4])
@pytest.mark.parametrize("n,out,E,T,k,x_slots", [
    (512, 96, 16, 64, 6, 1),     # ~24 tokens per expert: two token tiles
    (2048, 272, 5, 77, 2, 2),    # rows past a 256-row block, per-pair input
    (4096, 64, 8, 40, 3, 1),     # two activation chunks of 2048
    (4096, 256, 4, 100, 2, 2),   # ~50 tokens per expert: two passes over k
    (2048, 16, 12, 3, 6, 6),     # most experts idle
    (512, 768, 160, 80, 4, 1),   # more row blocks than workgroups: runs span several experts
])
def test_fused_prefill_matches_oracle(fmt, n, out, E, T, k, x_slots):
    seed = 1000 + fmt + n // 256 + out + T
    announce(f"fused prefill fmt={fmt} n={n} out={out} E={E} T={T} k={k} slots={x_slots}")
    w, s = _weights(fmt, E, out, n, seed)
    values, grid = synth.values_table(seed + 1), synth.ternary_grid(seed + 2)
    x = bf16_round(synth.normal((T, x_slots, n), seed + 3))
    ids = synth.topk_ids(T, k, E, seed + 4)
    y = q.moe_prefill_fused(w, to_dev(x, torch.bfloat16), to_dev(ids), values, to_dev(grid),
                            x_slots=x_slots).cpu().numpy()
    ref_b = oracle.moe(fmt, s, E, out, n, x, ids, values, grid, x_slots=x_slots, w_bf16=True)
    err = rel_err_per_vector(y, ref_b)
    assert np.all(err <= TOL_SAME_WEIGHTS), err.max()
    ref = oracle.moe(fmt, s, E, out, n, x, ids, values, grid, x_slots=x_slots)
    assert np.all(rel_err_per_vector(y, ref) <= TOL_BF16)


def test_fused_prefill_general_table_invalid_ids_and_two_pass_agreement():
    fmt, n, out, E, T, k = K, 2048, 128, 6, 30, 4
    w, s = _weights(fmt, E, out, n, 1100)
    values = (synth.values_table(1101) * 0.37).astype(np.float32)  # not integers: any float32 table
    x = bf16_round(synth.normal((T, 1, n), 1102))
    ids = synth.topk_ids(T, k, E, 1103)
    ids[3, 1] = -1
    ids[7, 0] = E + 2
    announce("fused prefill: float table, invalid ids, agreement with the two-pass prefill")
    sentinel = torch.full((T, k, out), 7.0, dtype=torch.float32, device="cuda")
    y = q.moe_prefill_fused(w, to_dev(x, torch.bfloat16), to_dev(ids), values, y=sentinel).cpu().numpy()
    assert np.all(np.isnan(y[3, 1])) and np.all(np.isnan(y[7, 0]))  # NaN rows, as on the per-pair path
    assert np.all(np.isfinite(y[(ids >= 0) & (ids < E)]))
    valid = ids >= 0
    valid &= ids < E
    ref_b = oracle.moe(fmt, s, E, out, n, x, np.where(valid, ids, 0), values, w_bf16=True)
    assert np.all(rel_err_per_vector(y[valid], ref_b[valid]) <= TOL_SAME_WEIGHTS)
    y2 = q.moe_prefill(w, to_dev(x, torch.bfloat16), to_dev(ids), values).cpu().numpy()
    assert np.all(rel_err_per_vector(y[valid], y2[valid].astype(np.float64)) <= TOL_SAME_WEIGHTS)


@pytest.mark.parametrize("fmt", [KS, K, R4])
def test_fused_prefill_skewed_routing(fmt):
    """One expert takes most pairs (several 32-token tiles), so the work plan
    spreads its row blocks over many workgroups while idle experts get none."""
    n, out, E, T, k = 2048, 1024, 8, 160, 2
    seed = 1200 + fmt
    announce(f"fused prefill skewed routing fmt={fmt}")
    w, s = _weights(fmt, E, out, n, seed)
    values, grid = synth.values_table(seed + 1), synth.ternary_grid(seed + 2)
    x = bf16_round(synth.normal((T, 1, n), seed + 3))
    ids = synth.topk_ids(T, k, E, seed + 4)
    hot = np.arange(T) % 8 != 7          # 140 of 160 tokens send their first pair to expert 0
    ids[hot, 0] = 0
    ids[hot, 1] = np.where(ids[hot, 1] == 0, 1, ids[hot, 1])
    ids[:, 1] = np.where(ids[:, 1] == 5, 3, ids[:, 1])   # expert 5 idle
    ids[:, 0] = np.where(ids[:, 0] == 5, 4, ids[:, 0])
    y = q.moe_prefill_fused(w, to_dev(x, torch.bfloat16), to_dev(ids), values, to_dev(grid)).cpu().numpy()
    ref_b = oracle.moe(fmt, s, E, out, n, x, ids, values, grid, w_bf16=True)
    assert np.all(rel_err_per_vector(y, ref_b) <= TOL_SAME_WEIGHTS)



@pytest.mark.parametrize("fmt", [KS, R4])
def test_fused_prefill_many_experts(fmt):
    """1500 experts: the work plan scans them in two chunks, the routing ranks
    with one wave"""
    n, out, E, T, k = 512, 16, 1500, 300, 6
    seed = 1800 + fmt
    announce(f"fused prefill many experts fmt={fmt}")
    w, s = _weights(fmt, E, out, n, seed)
    values, grid = synth.values_table(seed + 1), synth.ternary_grid(seed + 2)
    x = bf16_round(synth.normal((T, 1, n), seed + 3))
    ids = synth.topk_ids(T, k, E, seed + 4)
    y = q.moe_prefill_fused(w, to_dev(x, torch.bfloat16), to_dev(ids), values, to_dev(grid)).cpu().numpy()
    ref_b = oracle.moe(fmt, s, E, out, n, x, ids, values, grid, w_bf16=True)
    assert np.all(rel_err_per_vector(y, ref_b) <= TOL_SAME_WEIGHTS)
