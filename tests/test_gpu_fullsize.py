"""GPU parity at the workload's full sizes, in the launch configurations the
benchmark times: 256 experts, gate/up [4096, 4096] (gate and up stacked) and
down [4096, 2048] per expert, top-6 routing, bf16 activations.

The oracle cannot form every output at this size in seconds, so each test
checks sampled outputs one by one: for a sampled (token, slot, row) the
oracle packs that row from the wire itself, reconstructs it (float32 chain),
and forms the dot product in float64.  Bars per sampled element, relative to
the absolute-sum scale sum_k |w_k x_k| of that element: 1e-3 for the int8
fixed-point matvecs (per-vector bar of the path), 1e-4 for the fused prefill
against the bf16-rounded weights (its only difference is float32
summation order), bit-exact for the producer's bf16 rows.

Inputs: `synth.wire_experts` (one drawn expert, every other expert a copy
with its non-scale bytes XORed by a byte of its own), so the full stacked
tensors are built in seconds while every expert differs."""
import numpy as np
import pytest
import torch

import oracle
import synth
import dequant_iqk_moe_amd as q
from gpu_common import announce, to_dev

pytestmark = pytest.mark.gpu

KS, K, R4 = 1, 2, 3
E, H, I, TOPK = 256, 4096, 2048, 6
PROJ = {"gate_up": (2 * I, H, 1), "down": (H, I, TOPK)}


class Full:
    """one projection at full size: the wire (host), the GPU weights and
    oracle access to single rows"""

    def __init__(self, fmt, proj, seed):
        self.fmt, self.proj = fmt, proj
        self.out, self.n, self.slots = PROJ[proj]
        self.wire = synth.wire_experts(fmt, E, self.out, self.n, seed)
        self.w = q.Weights.from_wire(fmt, E, self.out, self.n, self.wire)
        self.rb = synth.row_bytes(fmt, self.n)
        self.values = synth.values_table(seed + 1)
        self.grid = synth.ternary_grid(seed + 2)
        self.grid_dev = to_dev(self.grid)

    def row(self, e, r, dtype=oracle.F32):
        """row r of expert e through the oracle (packed from its own wire bytes)"""
        R = e * self.out + r
        g = 4 if self.fmt == R4 else 1  # IQ1_S_R4 wire comes in four-row groups
        r0 = R - R % g
        wrows = self.wire[r0 * self.rb:(r0 + g) * self.rb]
        s = oracle.pack(self.fmt, wrows, g, self.n)
        return oracle.dequant(self.fmt, s, g, self.n, self.values, self.grid, dtype, r0=R - r0, nr=1)[0]


def _check_sampled(F, x, ids, y, rng, nsamp, tol, w_dtype=oracle.F32):
    """sampled outputs of y [T, k, out] against the oracle"""
    T, k = ids.shape
    yv = y.cpu().numpy()
    worst = 0.0
    for _ in range(nsamp):
        t, j, r = int(rng.integers(T)), int(rng.integers(k)), int(rng.integers(F.out))
        wr = F.row(int(ids[t, j]), r, w_dtype)
        if w_dtype == oracle.BF16:  # bf16 bit patterns -> their float values
            wr = (wr.astype(np.uint32) << 16).view(np.float32)
        wr = wr.astype(np.float64)
        xx = (x[t, 0] if F.slots == 1 else x[t, j]).astype(np.float64)
        ref = float(wr @ xx)
        scale = float(np.abs(wr) @ np.abs(xx))
        worst = max(worst, abs(float(yv[t, j, r]) - ref) / max(scale, 1e-30))
    assert worst <= tol, worst
    return worst


def _inputs(F, T, seed):
    x = torch.from_numpy(synth.normal((T, F.slots, F.n), seed)).to(torch.bfloat16)
    ids = synth.topk_ids(T, TOPK, E, seed + 1)
    return x, ids


@pytest.mark.parametrize("proj", ["gate_up", "down"])
@pytest.mark.parametrize("fmt", [KS, K, R4])
def test_fullsize(fmt, proj):
    """every path on one full-size projection (built once): decode matvec at
    T = 1 (and 8 for IQ2_KS), grouped matvec at T = 64, fused prefill at
    T = 512, producer rows"""
    announce(f"full-size fmt={fmt} {proj}: building the stacked weights")
    F = Full(fmt, proj, 3000 + 10 * fmt + (0 if proj == "gate_up" else 5))
    for T in ((1, 8) if fmt == KS else (1,)):
        announce(f"full-size decode matvec fmt={fmt} {proj} T={T}")
        x, ids = _inputs(F, T, 3100 + T)
        y = q.moe_gemv(F.w, x.cuda(), to_dev(ids), F.values, F.grid_dev, x_slots=F.slots)
        _check_sampled(F, x.float().numpy(), ids, y, np.random.default_rng(T), 48, 1e-3)

    announce(f"full-size grouped matvec fmt={fmt} {proj} T=64")
    x, ids = _inputs(F, 64, 3300)
    y = q.moe_gemv_grouped(F.w, x.cuda(), to_dev(ids), F.values, F.grid_dev, x_slots=F.slots)
    _check_sampled(F, x.float().numpy(), ids, y, np.random.default_rng(8), 64, 1e-3)

    announce(f"full-size fused prefill fmt={fmt} {proj} T=512")
    x, ids = _inputs(F, 512, 3200)
    y = q.moe_prefill_fused(F.w, x.cuda(), to_dev(ids), F.values, F.grid_dev, x_slots=F.slots)
    # the same bf16 weights as the producer: the bar is float32 summation order
    _check_sampled(F, x.float().numpy(), ids, y, np.random.default_rng(7), 64, 1e-4, oracle.BF16)
    del y

    announce(f"full-size producer fmt={fmt} {proj}")
    dense = q.dequant(F.w, F.values, F.grid_dev, torch.bfloat16)  # [E * out, n], the prefill's dense copy
    rng = np.random.default_rng(9)
    for _ in range(32):
        e, r = int(rng.integers(E)), int(rng.integers(F.out))
        got = dense[e * F.out + r].cpu().view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(got, F.row(e, r, oracle.BF16))
    del dense, F
    torch.cuda.empty_cache()
