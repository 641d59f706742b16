"""GPU parity at the workload's full sizes, in the launch configurations the
benchmark times: 256 experts, gate/up [4096, 4096] (gate and up stacked) and
down [4096, 2048] per expert, top-6 routing, bf16 activations.

Whole output vectors are compared with the oracle: for a chosen (token,
slot) pair the oracle packs that pair's expert from the wire itself and
forms the full output row set y[t, j, :] (float32 chain per weight, float64
sums).  Bars per output vector: ||y - y_exact|| / ||y_exact|| <= 1e-3 for
the matvecs (fp32 accumulation), <= 1e-4 for the fused prefill against the
bf16-rounded weights it multiplies with (its only difference from the
oracle is float32 summation order) and <= 2e-2 against the float32
weights; the producer's bf16 rows bit-exact.  Vectors: all six pairs of a
one-token call, eight whole pairs of every larger call.

The one-token layer's glue modes (SwiGLU epilogue, router-weighted
combine) get the same whole-vector comparison on the full IQ2_K tensors.

Inputs: `synth.wire_experts` (one drawn expert, every other expert a copy
with its non-scale bytes XORed by a byte of its own), so the full stacked
tensors are built in seconds while every expert differs."""
import concurrent.futures as cf

import numpy as np
import pytest
import torch

import oracle
import synth
import dequant_iqk_moe_amd as q
from gpu_common import TOL_BF16, TOL_GEMV, announce, bf16_storage_excess, rel_err_per_vector, to_dev

pytestmark = pytest.mark.gpu

KS, K, R4 = 1, 2, 3
E, H, I, TOPK = 256, 4096, 2048, 6
PROJ = {"gate_up": (2 * I, H, 1), "down": (H, I, TOPK)}
TOL_FUSED_BF16W = 1e-4
_POOL = cf.ThreadPoolExecutor(max_workers=8)  # the oracle's C calls release the GIL


class Full:
    """one projection at full size: the wire (host), the GPU weights and
    oracle access to single experts"""

    def __init__(self, fmt, proj, seed):
        self.fmt, self.proj = fmt, proj
        self.out, self.n, self.slots = PROJ[proj]
        self.wire = synth.wire_experts(fmt, E, self.out, self.n, seed)
        self.w = q.Weights.from_wire(fmt, E, self.out, self.n, self.wire)
        self.rb = synth.row_bytes(fmt, self.n)
        self.values = synth.values_table(seed + 1)
        self.grid = synth.ternary_grid(seed + 2)
        self.grid_dev = to_dev(self.grid)
        self._streams = {}

    def expert_streams(self, e):
        """expert e's [out, n] streams, packed by the oracle from its own wire bytes"""
        if e not in self._streams:
            span = self.out * self.rb
            self._streams[e] = oracle.pack(self.fmt, self.wire[e * span:(e + 1) * span], self.out, self.n)
        return self._streams[e]

    def vector(self, e, xvec, w_bf16=False):
        """y = W_e x for one whole output vector (float64, [out])"""
        y = oracle.moe(self.fmt, self.expert_streams(e), 1, self.out, self.n, xvec.reshape(1, 1, self.n),
                       np.zeros((1, 1), np.int32), self.values, self.grid, w_bf16=w_bf16)
        return y[0, 0]

    def row(self, e, r, dtype=oracle.F32):
        """row r of expert e through the oracle"""
        return oracle.dequant(self.fmt, self.expert_streams(e), self.out, self.n, self.values, self.grid, dtype,
                              r0=r, nr=1)[0]


def _pairs(T, rng, count=8):
    """all pairs of a one-token call, else `count` distinct random (t, j)"""
    if T == 1:
        return [(0, j) for j in range(TOPK)]
    flat = rng.choice(T * TOPK, size=count, replace=False)
    return [(int(p) // TOPK, int(p) % TOPK) for p in flat]


def _check_vectors(F, x, ids, y, pairs, bars):
    """whole vectors y[t, j, :] against the oracle; bars: [(w_bf16, tol)]"""
    yv = y.cpu().numpy()
    for w_bf16, tol in bars:
        xs = [(x[t, 0] if F.slots == 1 else x[t, j]) for t, j in pairs]
        for (t, j), e in zip(pairs, (int(ids[t, j]) for t, j in pairs)):
            F.expert_streams(e)  # packed once, before the threads read the cache
        refs = list(_POOL.map(lambda a: F.vector(int(ids[a[0][0], a[0][1]]), a[1], w_bf16), zip(pairs, xs)))
        got = np.stack([yv[t, j] for t, j in pairs])
        err = rel_err_per_vector(got, np.stack(refs))
        assert np.all(err <= tol), (w_bf16, tol, err.max())


def _inputs(F, T, seed):
    x = torch.from_numpy(synth.normal((T, F.slots, F.n), seed)).to(torch.bfloat16)
    ids = synth.topk_ids(T, TOPK, E, seed + 1)
    return x, ids


@pytest.mark.parametrize("proj", ["gate_up", "down"])
@pytest.mark.parametrize("fmt", [KS, K, R4])
def test_fullsize(fmt, proj):
    """every path on one full-size projection (built once): decode matvec at
    T = 1 and 8, grouped matvec at T = 64, fused prefill at T = 512,
    producer rows"""
    announce(f"full-size fmt={fmt} {proj}: building the stacked weights")
    F = Full(fmt, proj, 3000 + 10 * fmt + (0 if proj == "gate_up" else 5))
    for T in (1, 8):
        announce(f"full-size decode matvec fmt={fmt} {proj} T={T}")
        x, ids = _inputs(F, T, 3100 + T)
        y = q.moe_gemv(F.w, x.cuda(), to_dev(ids), F.values, F.grid_dev, x_slots=F.slots)
        _check_vectors(F, x.float().numpy(), ids, y, _pairs(T, np.random.default_rng(T)), [(False, TOL_GEMV)])

    announce(f"full-size grouped matvec fmt={fmt} {proj} T=64")
    x, ids = _inputs(F, 64, 3300)
    y = q.moe_gemv_grouped(F.w, x.cuda(), to_dev(ids), F.values, F.grid_dev, x_slots=F.slots)
    _check_vectors(F, x.float().numpy(), ids, y, _pairs(64, np.random.default_rng(8)), [(False, TOL_GEMV)])

    announce(f"full-size fused prefill fmt={fmt} {proj} T=512")
    x, ids = _inputs(F, 512, 3200)
    y = q.moe_prefill_fused(F.w, x.cuda(), to_dev(ids), F.values, F.grid_dev, x_slots=F.slots)
    _check_vectors(F, x.float().numpy(), ids, y, _pairs(512, np.random.default_rng(7)),
                   [(True, TOL_FUSED_BF16W), (False, TOL_BF16)])
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


def test_fullsize_layer_glue_modes():
    """The one-token layer the benchmark times, on the full stacked IQ2_K
    tensors: gate/up with the SwiGLU epilogue (every pair's whole h vector
    at the SwiGLU bar: the matvec's 1e-3 past the bf16 cast's half step),
    then down with the router-weighted combine on that h (the token's whole
    y vector at 1e-3 of sum_j |w_j| ||W_j h_j||); T = 1 and 4."""
    announce("full-size layer glue: building the stacked IQ2_K weights")
    Fg = Full(K, "gate_up", 3400)
    Fd = Full(K, "down", 3405)
    I = Fd.n
    for T in (1, 4):
        announce(f"full-size layer glue T={T}")
        x, ids = _inputs(Fg, T, 3500 + T)
        rw = np.random.default_rng(3600 + T).dirichlet(np.ones(TOPK), size=T).astype(np.float32)
        idd = to_dev(ids)
        h = q.moe_gemv_swiglu(Fg.w, x.cuda(), idd, Fg.values)
        # the combine takes this h; down's value table is its own (as the bench's layer)
        y = q.moe_gemv_combine(Fd.w, h, idd, to_dev(rw), Fd.values, x_slots=TOPK)
        hv = h.float().cpu().numpy()
        yv = y.cpu().numpy()
        xv = x.float().numpy()
        for t in range(T):
            for e in (int(v) for v in ids[t]):
                Fg.expert_streams(e)
                Fd.expert_streams(e)
            gu = list(_POOL.map(lambda j: Fg.vector(int(ids[t, j]), xv[t, 0]), range(TOPK)))
            h_ref = oracle.swiglu(np.stack(gu)[None])[0]                      # [k, I]
            assert np.all(bf16_storage_excess(hv[t], h_ref) <= TOL_GEMV)
            parts = np.stack(list(_POOL.map(lambda j: Fd.vector(int(ids[t, j]), hv[t, j]), range(TOPK))))
            y_ref = oracle.combine(parts[None], rw[t:t + 1])[0]
            scale = np.sum(np.abs(rw[t])[:, None] * np.linalg.norm(parts, axis=-1, keepdims=True))
            assert np.linalg.norm(yv[t] - y_ref) / scale <= TOL_GEMV
        assert h.shape == (T, TOPK, I)
    del Fg, Fd
    torch.cuda.empty_cache()
