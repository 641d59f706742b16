#!/usr/bin/env python3
"""Routed-expert decode benchmark on one MI355X.

Headline workload: IQ2_K routed MoE decode, 1 token, top-6 of 256 experts,
gate and up [2048, 4096] stored as one fused [4096, 4096] tensor per expert,
down [4096, 2048]; activation bf16 N(0,1); fp16 super-block scales
|N(0,1)| * 0.01; codes, scale indices and alphabet bits uniform ("mlx-iqk"
routed geometry).  One step = the gate/up matvec launch plus the down matvec
launch of one MoE layer's routed projections (the down input is a synthetic
bf16 [1, 6, 2048] tensor; the SwiGLU between them is outside this path).

Timing: inputs are resident in HBM before timing.  Weights are rotated over
8 independent pools (each step uses the next pool and fresh expert ids) so no
step can be served from the 256 MiB last-level cache.  S steps are captured
into one HIP graph and replayed; W warmup steps, then exactly K timed steps
between two synchronizations, HIP events on the launch stream.  Value =
algorithmic bytes (compressed bytes of the distinct selected experts + x + y)
per second.

`roofline` reports the dominant kernel (the gate/up matvec): algorithmic
bytes per launch over its average launch duration, from a graph of that
kernel alone.  `cells` (default on) adds every format x projection x token
count of the workload family, each with its deleted-decode floor and a plain
streaming read of the same byte count, plus the prefill rows at 512 tokens
(routing, dequantization producer, MFMA grouped GEMM, and the fused prefill
with the dequantization inside the MFMA GEMM; `--cells prefill` runs only
these).  `cpu_baseline`
times the CPU oracle on whole decode steps (about 10 s of CPU work).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
POOLS = 8
E, K, H, I = 256, 6, 4096, 2048
FMT_NAME = {1: "IQ2_KS", 2: "IQ2_K", 3: "IQ1_S_R4"}


def _parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    # 6000 steps (~0.1 s): the GPU raises its clocks over ~10-20 ms of load
    # after idling, so the timed steps start at the steady clock
    ap.add_argument("--warmup", type=int, default=6000)
    ap.add_argument("--cells", choices=["none", "all", "prefill"], default="all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=2)
    ap.add_argument("--mode", choices=["bench", "pmc", "sweep", "ceiling"], default="bench",
                    help="ceiling: plain HBM writes at the dequantization producer's output sizes beside "
                         "the bf16 producers of every member (the producer's write ceiling); "
                         "pmc: only launch the headline gate/up matvec 64 times plus two calibration "
                         "kernels of known traffic (a 256 MiB streaming read and a 256 MiB fill), "
                         "for hardware-counter runs; sweep: decode <-> prefill crossover over "
                         "T = 1..512 for every format and projection (one JSON line each)")
    return ap.parse_args()


def _host_cpu():
    """CPU model and logical core count of the host the baseline ran on"""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "logical_cores": os.cpu_count()}


def log(msg):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


class Pools:
    """Expert-stacked stream tensors of one projection, replicated over pools."""

    def __init__(self, q, torch, fmt, out, n, seed, pools=POOLS):
        import synth
        wire = synth.wire(fmt, E * out, n, seed)
        self.wire = wire  # the oracle packs what it needs from the wire itself
        base = torch.from_numpy(q.pack_relayout(fmt, wire, E * out, n)).cuda()
        self.w = [q.Weights(fmt, E, out, n, base)] + [q.Weights(fmt, E, out, n, base.clone()) for _ in range(pools - 1)]
        self.fmt, self.out, self.n = fmt, out, n
        self.row_bytes = q.row_bytes(fmt, n)

    def bytes_for(self, ids: np.ndarray) -> int:
        """algorithmic weight bytes: every distinct selected expert once"""
        return len(np.unique(ids)) * self.out * self.row_bytes


# Secondary cells run after host-side work (validation, oracle rows) that
# leaves the GPU idle and its clocks lowered; each is run for this long
# (untimed) before it is timed.  Measured: a 0.5 ms fused prefill call takes
# ~20 % longer, and a T=1 decode launch ~5 % longer, in the first ~10 ms
# after an idle second.
CLOCK_RAMP_S = 0.05
# Pricing gates ("mlx-iqk" package description, "Pricing"): a decode cell
# passes at <= 1.25x its deleted-decode floor, and its floor arm is only
# trusted while it streams within [0.85, 1.05] x a plain read of the same
# bytes measured in the same session.
RATIO_BAR = 1.25
BAND = (0.85, 1.05)
PREFILL_REPS = 50  # calls per timed prefill arm (medians over three alternating rounds where arms alternate)


def ramp_clocks(torch, run):
    """run() untimed for CLOCK_RAMP_S; returns how many times it ran"""
    t0 = time.perf_counter()
    calls = 0
    while time.perf_counter() - t0 < CLOCK_RAMP_S:
        run()
        torch.cuda.synchronize()
        calls += 1
    return calls


def timed_graph(torch, fn, S, reps, warm_reps, ramp=True, info=None):
    """Capture S calls of fn(i) in one graph; replay; return ms per call.
    ramp=False keeps the warm-up to exactly warm_reps replays.  `info`
    (a dict) receives the untimed replays run before timing."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(S):  # eager pass: every launch is checked before capture
            fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(S):
            fn(i)
    for _ in range(warm_reps):
        g.replay()
    torch.cuda.synchronize()
    ramp_calls = ramp_clocks(torch, g.replay) if ramp else 0
    # one more untimed replay, not waited for: the GPU is busy with it while
    # the start event and the timed replays are queued, so the idle GPU's
    # wake-up and the first launch's latency stay out of the timed region
    g.replay()
    if info is not None:
        info["untimed_replays"] = warm_reps + ramp_calls + 1
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * S)


def timed_eager(torch, fn, reps, warm):
    for i in range(warm):
        fn(i)
    torch.cuda.synchronize()
    ramp_clocks(torch, lambda: fn(0))
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


class Ctx:
    def __init__(self, q, torch, seed):
        import synth
        self.q, self.torch = q, torch
        self.values = synth.values_table(seed + 1)
        self.grid_host = synth.ternary_grid(seed + 4)
        self.grid = torch.from_numpy(self.grid_host).cuda()
        self.sbuf = None
        self.ssink = torch.zeros(1 << 14, dtype=torch.int32, device="cuda")

    def stream_ms(self, nbytes, S, reps, warm):
        nb = int(nbytes) // 16 * 16
        slots = 16
        need = nb * slots
        if self.sbuf is None or self.sbuf.numel() < need:
            self.sbuf = None
            self.sbuf = self.torch.empty(need, dtype=self.torch.uint8, device="cuda")
            self.sbuf.fill_(1)

        def sread(i):
            self.q.stream_read(self.sbuf[(i % slots) * nb:(i % slots + 1) * nb], self.ssink)

        return timed_graph(self.torch, sread, S, reps, warm)


def oracle_moe_subset(oracle, fmt, wire, out, n, x, ids, values, grid_host=None, x_slots=1):
    """the oracle's routed product over only the selected experts, packed by
    the oracle from the wire (ids remapped onto the subset)"""
    import synth
    rb = synth.row_bytes(fmt, n)
    experts = sorted(set(int(e) for e in np.asarray(ids).ravel()))
    remap = {e: i for i, e in enumerate(experts)}
    ids2 = np.vectorize(remap.get)(np.asarray(ids)).astype(np.int32)
    sub = np.concatenate([wire[e * out * rb:(e + 1) * out * rb] for e in experts])
    streams = oracle.pack(fmt, sub, len(experts) * out, n)
    return oracle.moe(fmt, streams, len(experts), out, n, x, ids2, values, grid_host, x_slots=x_slots)


def layer_cell(ctx, gate_up, down, x, S, reps, warm, seed):
    """One MoE layer's routed experts at T=1 with the glue fused: gate/up
    matvec + SwiGLU (bf16 h), then down matvec + router-weighted combine
    (y [1, hidden]).  Validated in full against the oracle first."""
    import synth
    import oracle
    q, torch = ctx.q, ctx.torch
    T = 1
    ids_host = [synth.topk_ids(T, K, E, seed * 1000 + i) for i in range(S)]
    ids = [torch.from_numpy(a).cuda() for a in ids_host]
    rw_host = np.random.default_rng(seed).dirichlet(np.ones(K), size=T).astype(np.float32)
    rw = torch.from_numpy(rw_host).cuda()
    hbuf = torch.empty((T, K, I), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")
    q.moe_gemv_swiglu(gate_up.w[0], x, ids[0], ctx.values, h=hbuf)
    q.moe_gemv_combine(down.w[0], hbuf, ids[0], rw, ctx.values, y=y)
    torch.cuda.synchronize()
    xv = x.float().cpu().numpy().reshape(T, 1, H)
    gu = oracle_moe_subset(oracle, q.IQ2_K, gate_up.wire, 2 * I, H, xv, ids_host[0], ctx.values)
    h_ref = oracle.swiglu(gu)
    h_gpu = hbuf.float().cpu().numpy()
    err_h = float(np.max(np.linalg.norm(h_gpu - h_ref, axis=-1) / np.linalg.norm(h_ref, axis=-1)))
    parts = oracle_moe_subset(oracle, q.IQ2_K, down.wire, H, I, h_gpu, ids_host[0], ctx.values, x_slots=K)
    y_ref = oracle.combine(parts, rw_host)
    scale = np.sum(np.abs(rw_host)[:, :, None] * np.linalg.norm(parts, axis=-1, keepdims=True), axis=1)[:, 0]
    err_y = float(np.max(np.linalg.norm(y.cpu().numpy() - y_ref, axis=-1) / scale))

    def run(i):
        p = i % POOLS
        q.moe_gemv_swiglu(gate_up.w[p], x, ids[i], ctx.values, h=hbuf)
        q.moe_gemv_combine(down.w[p], hbuf, ids[i], rw, ctx.values, y=y)

    ms = timed_graph(torch, run, S, reps, warm)
    nbytes = float(np.mean([gate_up.bytes_for(a) + down.bytes_for(a) for a in ids_host])) + \
        x.numel() * 2 + 2 * hbuf.numel() * 2 + y.numel() * 4 + rw.numel() * 4
    return {"cell": "IQ2_K MoE layer T=1: gate/up+SwiGLU, down+combine", "kind": "layer",
            "us": round(ms * 1e3, 3), "bytes": int(nbytes), "GBps": round(nbytes / (ms * 1e-3) / 1e9, 2),
            "tokens_per_s": round(T / (ms * 1e-3), 1), "validation_h": err_h, "validation_y": err_y}


def decode_cell(ctx, pool, T, proj, S, reps, warm, seed):
    """one matvec cell: kernel time, floor time, stream-read time for the same bytes"""
    import synth
    import oracle
    q, torch = ctx.q, ctx.torch
    slots = 1 if proj == "gate_up" else K
    ids_host = [synth.topk_ids(T, K, E, seed * 1000 + i) for i in range(S)]
    ids = [torch.from_numpy(a).cuda() for a in ids_host]
    x = torch.from_numpy(synth.normal((T, slots, pool.n), seed + 7)).to(torch.bfloat16).cuda()
    y = torch.empty((T, K, pool.out), dtype=torch.float32, device="cuda")
    sink = torch.empty((T, K, pool.out), dtype=torch.int32, device="cuda")
    grid = ctx.grid if pool.fmt == 3 else None
    q.moe_gemv(pool.w[0], x, ids[0], ctx.values, grid, x_slots=slots, y=y)
    torch.cuda.synchronize()
    worst = validate_vectors(oracle, q, pool, ids_host[0], x.float().cpu().numpy(), y, slots, ctx.values,
                             ctx.grid_host, sample_pairs(T, K, np.random.default_rng(seed)))
    if worst > 1e-3:
        raise RuntimeError(f"{FMT_NAME[pool.fmt]} {proj} T={T}: validation failed, per-vector error {worst:.3e}")

    def run(i):
        q.moe_gemv(pool.w[i % POOLS], x, ids[i], ctx.values, grid, x_slots=slots, y=y)

    def run_floor(i):
        q.floor_gemv(pool.w[i % POOLS], x, ids[i], ctx.values, grid, x_slots=slots, sink=sink)

    # decode and floor arms alternate (A B A B A B); medians
    arms = {"decode": [], "floor": []}
    for _ in range(3):
        arms["decode"].append(timed_graph(torch, run, S, reps, warm))
        arms["floor"].append(timed_graph(torch, run_floor, S, reps, warm))
    ms, ms_floor = float(np.median(arms["decode"])), float(np.median(arms["floor"]))
    nbytes = float(np.mean([pool.bytes_for(a) for a in ids_host])) + x.numel() * 2 + y.numel() * 4
    ms_stream = ctx.stream_ms(nbytes, S, reps, warm)
    gbs = nbytes / (ms * 1e-3) / 1e9
    band = ms_stream / ms_floor
    return {"cell": f"{FMT_NAME[pool.fmt]} {proj} T={T}", "kind": "decode", "us": round(ms * 1e3, 3),
            "bytes": int(nbytes), "GBps": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
            "floor_us": round(ms_floor * 1e3, 3), "ratio_to_floor": round(ms / ms_floor, 3),
            "ratio_ok": ms / ms_floor <= RATIO_BAR,
            "stream_read_us": round(ms_stream * 1e3, 3),
            "floor_rate_vs_stream": round(band, 3), "band_ok": BAND[0] <= band <= BAND[1],
            "tokens_per_s": round(T / (ms * 1e-3), 1), "validation_worst": worst}


def prefill_cells(ctx, fmt, seed):
    """routing + producer + grouped GEMM at 512 tokens for gate/up and down"""
    import synth
    import oracle
    q, torch = ctx.q, ctx.torch
    T = 512
    out = []
    ids_h = synth.topk_ids(T, K, E, seed + 11)
    ids = torch.from_numpy(ids_h).cuda()
    counts, offsets, perm = q.route(ids, E)
    route_ms = timed_eager(torch, lambda i: q.route(ids, E), PREFILL_REPS, 5)
    total_ms = route_ms
    fused_total_ms = 0.0
    out.append({"cell": f"{FMT_NAME[fmt]} prefill route T=512", "kind": "route", "us": round(route_ms * 1e3, 3)})
    grid = ctx.grid if fmt == 3 else None
    for proj, (rows, n) in (("gate_up", (2 * I, H)), ("down", (H, I))):
        slots = 1 if proj == "gate_up" else K
        wire = synth.wire(fmt, E * rows, n, seed + (1 if proj == "gate_up" else 2))
        w = q.Weights(fmt, E, rows, n, torch.from_numpy(q.pack_relayout(fmt, wire, E * rows, n)).cuda())
        dense = torch.empty((E, rows, n), dtype=torch.bfloat16, device="cuda")
        x = torch.from_numpy(synth.normal((T, slots, n), seed + 5)).to(torch.bfloat16).cuda()
        y = torch.zeros((T, K, rows), dtype=torch.float32, device="cuda")
        q.dequant(w, ctx.values, grid, torch.bfloat16, out=dense.view(E * rows, n))
        q.grouped_gemm(dense, x, T, K, offsets, perm, x_slots=slots, y=y)
        torch.cuda.synchronize()
        # validation: whole output vectors of 8 pairs against the oracle's
        # float32-weight product (bf16 weights: 2e-2)
        pool = _WireProj(fmt, rows, n, wire)
        vpairs = sample_pairs(T, K, np.random.default_rng(seed))
        xv = x.float().cpu().numpy()
        worst = validate_vectors(oracle, q, pool, ids_h, xv, y, slots, ctx.values, ctx.grid_host, vpairs)
        if worst > 2e-2:
            raise RuntimeError(f"{FMT_NAME[fmt]} prefill {proj}: validation failed, per-vector error {worst:.3e}")
        wbytes = E * rows * q.row_bytes(fmt, n)
        dbytes = E * rows * n * 2
        dv = dense.view(E * rows, n)
        # producer, floor and plain writes of the same output bytes (the
        # write ceiling: one 1 KiB store per wave; and the producer's own
        # store shape, eight per wave) alternate, three rounds each, medians
        # of 50 calls
        arms = {"prod": [], "floor": [], "write": [], "write8": []}
        for _ in range(3):
            arms["prod"].append(timed_eager(torch, lambda i: q.dequant(w, ctx.values, grid, torch.bfloat16, out=dv),
                                            PREFILL_REPS, 2))
            arms["floor"].append(timed_eager(torch, lambda i: q.floor_dequant(w, torch.bfloat16, out=dv),
                                             PREFILL_REPS, 2))
            arms["write"].append(timed_eager(torch, lambda i: q.stream_write(dv, 0x3F803F80), PREFILL_REPS, 2))
            arms["write8"].append(timed_eager(torch, lambda i: q.stream_write(dv, 0x3F803F80, runs=8), PREFILL_REPS, 2))
        prod_ms, floor_ms = float(np.median(arms["prod"])), float(np.median(arms["floor"]))
        write_ms, write8_ms = float(np.median(arms["write"])), float(np.median(arms["write8"]))
        q.dequant(w, ctx.values, grid, torch.bfloat16, out=dv)  # the floor left raw words in the dense copy
        pbytes = wbytes + dbytes
        pg = pbytes / (prod_ms * 1e-3) / 1e9
        out.append({"cell": f"{FMT_NAME[fmt]} prefill producer {proj}", "kind": "producer",
                    "us": round(prod_ms * 1e3, 1), "bytes": int(pbytes), "GBps": round(pg, 1),
                    "frac_hbm": round(pg / HBM_PEAK_GBS, 4), "floor_us": round(floor_ms * 1e3, 1),
                    "ratio_to_floor": round(prod_ms / floor_ms, 3),
                    "write_ceiling_us": round(write_ms * 1e3, 1),
                    "write_ceiling_GBps": round(dbytes / (write_ms * 1e-3) / 1e9, 1),
                    "vs_write_ceiling": round(write_ms / prod_ms, 3),
                    "same_shape_write_us": round(write8_ms * 1e3, 1),
                    "vs_same_shape_write": round(write8_ms / prod_ms, 3)})
        gemm_ms = timed_eager(torch, lambda i: q.grouped_gemm(dense, x, T, K, offsets, perm, x_slots=slots, y=y),
                              PREFILL_REPS, 2)
        gbytes = dbytes + x.numel() * 2 + y.numel() * 4
        flops = 2.0 * T * K * rows * n
        gg = gbytes / (gemm_ms * 1e-3) / 1e9
        tf = flops / (gemm_ms * 1e-3) / 1e12
        out.append({"cell": f"{FMT_NAME[fmt]} prefill grouped GEMM {proj}", "kind": "gemm",
                    "us": round(gemm_ms * 1e3, 1), "bytes": int(gbytes), "GBps": round(gg, 1),
                    "frac_hbm": round(gg / HBM_PEAK_GBS, 4), "TFLOPs": round(tf, 2),
                    "mfma_util": round(tf / BF16_PEAK_TFLOPS, 4), "validation_worst": worst})
        total_ms += prod_ms + gemm_ms
        del dense, dv
        torch.cuda.empty_cache()
        # the same product with the dequantization inside the MFMA GEMM (route + plan + one kernel)
        ws = torch.empty(q.prefill_fused_workspace_bytes(w, T, K), dtype=torch.uint8, device="cuda")
        yf = torch.zeros_like(y)
        q.moe_prefill_fused(w, x, ids, ctx.values, grid, x_slots=slots, workspace=ws, y=yf)
        torch.cuda.synchronize()
        fused_vs_two_pass = float((yf - y).abs().max() / y.abs().max().clamp_min(1e-30))
        # the fused product multiplies the same bf16 weights: 1e-4 against that product
        worst_f = validate_vectors(oracle, q, pool, ids_h, xv, yf, slots, ctx.values, ctx.grid_host, vpairs,
                                   w_bf16=True)
        if worst_f > 1e-4:
            raise RuntimeError(f"{FMT_NAME[fmt]} fused prefill {proj}: validation failed, {worst_f:.3e}")
        fused_ms = timed_eager(torch, lambda i: q.moe_prefill_fused(w, x, ids, ctx.values, grid, x_slots=slots,
                                                                      workspace=ws, y=yf), PREFILL_REPS, 2)
        fbytes = wbytes + x.numel() * 2 + y.numel() * 4
        out.append({"cell": f"{FMT_NAME[fmt]} prefill fused {proj}", "kind": "fused",
                    "us": round(fused_ms * 1e3, 1), "bytes": int(fbytes),
                    "GBps": round(fbytes / (fused_ms * 1e-3) / 1e9, 1),
                    "TFLOPs": round(flops / (fused_ms * 1e-3) / 1e12, 2),
                    "mfma_util": round(flops / (fused_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                    "weights_per_s": round(E * rows * n / (fused_ms * 1e-3), 1),
                    "max_rel_diff_vs_two_pass": fused_vs_two_pass, "validation_worst_bf16_weights": worst_f})
        fused_total_ms += fused_ms
        del w, y, yf, ws
        torch.cuda.empty_cache()
    out.append({"cell": f"{FMT_NAME[fmt]} prefill total (route + 2 x (producer + GEMM))", "kind": "prefill",
                "us": round(total_ms * 1e3, 1), "tokens_per_s": round(T / (total_ms * 1e-3), 1)})
    out.append({"cell": f"{FMT_NAME[fmt]} prefill total fused (2 x (route + fused GEMM))", "kind": "prefill",
                "us": round(fused_total_ms * 1e3, 1), "tokens_per_s": round(T / (fused_total_ms * 1e-3), 1)})
    return out


def prefill_layer_cell(ctx, seed):
    """One MoE layer's routed experts at 512 tokens through the fused
    prefill: gate/up (route + fused GEMM), SwiGLU to bf16 h, down (route +
    fused GEMM) and the router-weighted combine to y [512, hidden].  Two
    sampled tokens are checked against the oracle chain first."""
    import synth
    import oracle
    q, torch = ctx.q, ctx.torch
    T, fmt = 512, q.IQ2_K
    wgu = synth.wire(fmt, E * 2 * I, H, seed + 1)
    wdn = synth.wire(fmt, E * H, I, seed + 2)
    gu = q.Weights(fmt, E, 2 * I, H, torch.from_numpy(q.pack_relayout(fmt, wgu, E * 2 * I, H)).cuda())
    dn = q.Weights(fmt, E, H, I, torch.from_numpy(q.pack_relayout(fmt, wdn, E * H, I)).cuda())
    ids_h = synth.topk_ids(T, K, E, seed + 3)
    ids = torch.from_numpy(ids_h).cuda()
    rw_h = np.random.default_rng(seed + 4).dirichlet(np.ones(K), size=T).astype(np.float32)
    rw = torch.from_numpy(rw_h).cuda()
    x = torch.from_numpy(synth.normal((T, 1, H), seed + 5)).to(torch.bfloat16).cuda()
    ws = torch.empty(q.prefill_fused_workspace_bytes(gu, T, K), dtype=torch.uint8, device="cuda")
    y_gu = torch.empty((T, K, 2 * I), dtype=torch.float32, device="cuda")
    h = torch.empty((T, K, I), dtype=torch.bfloat16, device="cuda")
    y_dn = torch.empty((T, K, H), dtype=torch.float32, device="cuda")
    y = torch.empty((T, H), dtype=torch.float32, device="cuda")

    def run(i):
        q.moe_prefill_fused(gu, x, ids, ctx.values, workspace=ws, y=y_gu)
        q.swiglu(y_gu, h=h)
        q.moe_prefill_fused(dn, h, ids, ctx.values, x_slots=K, workspace=ws, y=y_dn)
        q.combine(y_dn, rw, yc=y)

    run(0)
    torch.cuda.synchronize()
    # the oracle chain on two tokens (bf16 weights, as the prefill multiplies with)
    worst_h, worst_y = 0.0, 0.0
    for t in (3, 300):
        xt = x[t:t + 1].float().cpu().numpy()
        sel = ids_h[t:t + 1]
        experts = sorted(set(int(e) for e in sel.ravel()))
        remap = {e: j for j, e in enumerate(experts)}
        sel2 = np.vectorize(remap.get)(sel).astype(np.int32)
        rbg, rbd = q.row_bytes(fmt, H), q.row_bytes(fmt, I)
        sg = oracle.pack(fmt, np.concatenate([wgu[e * 2 * I * rbg:(e + 1) * 2 * I * rbg] for e in experts]),
                         len(experts) * 2 * I, H)
        sd = oracle.pack(fmt, np.concatenate([wdn[e * H * rbd:(e + 1) * H * rbd] for e in experts]),
                         len(experts) * H, I)
        h_ref = oracle.swiglu(oracle.moe(fmt, sg, len(experts), 2 * I, H, xt, sel2, ctx.values, w_bf16=True))
        h_gpu = h[t:t + 1].float().cpu().numpy()
        worst_h = max(worst_h, float(np.max(np.linalg.norm(h_gpu - h_ref, axis=-1) /
                                            np.linalg.norm(h_ref, axis=-1))))
        parts = oracle.moe(fmt, sd, len(experts), H, I, h_gpu, sel2, ctx.values, x_slots=K, w_bf16=True)
        y_ref = oracle.combine(parts, rw_h[t:t + 1])
        scale = float(np.sum(np.abs(rw_h[t]) * np.linalg.norm(parts[0], axis=-1)))
        worst_y = max(worst_y, float(np.linalg.norm(y[t].cpu().numpy() - y_ref[0]) / scale))
    ms = timed_eager(torch, run, PREFILL_REPS, 2)
    del gu, dn, ws, y_gu, h, y_dn, y
    torch.cuda.empty_cache()
    return {"cell": "IQ2_K MoE layer T=512 prefill: fused gate/up, SwiGLU, fused down, combine", "kind": "prefill",
            "us": round(ms * 1e3, 1), "tokens_per_s": round(T / (ms * 1e-3), 1), "validation_h": worst_h,
            "validation_y": worst_y}


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "gemv_iqk2k_gate_up_t1_traffic.md")
GEMV_SOURCES = ("dequant_iqk_moe_amd/csrc/iqk_gemv.hip", "dequant_iqk_moe_amd/csrc/iqk_device.h",
                "dequant_iqk_moe_amd/csrc/iqk_internal.h")


def _traffic_fields():
    """the committed FETCH_SIZE/WRITE_SIZE summary's fields, or None when the
    matvec sources changed since the counters were taken"""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines()
                  if line.startswith(("traffic_bytes_per_launch: ", "floor_fetch_bytes_per_launch: ",
                                      "algorithmic_bytes_per_launch: ", "source_sha256: ")))
    if fields.get("source_sha256", "").strip() != gemv_source_hash():
        return None
    return fields


def measured_traffic():
    """HBM bytes per gate/up launch from the committed counter summary, or
    None when the kernel sources changed since it was taken."""
    f = _traffic_fields()
    return int(f["traffic_bytes_per_launch"]) if f else None


def deleted_load_check():
    """The pages' third pricing gate ("Pricing": no deleted-load signature):
    the floor arm must read what the decode reads.  From the same counter
    summary: the floor kernel's scaled FETCH_SIZE over the algorithmic bytes,
    ok at >= 0.98; None when the summary does not match the sources."""
    f = _traffic_fields()
    if not f or "floor_fetch_bytes_per_launch" not in f:
        return None
    ratio = int(f["floor_fetch_bytes_per_launch"]) / int(f["algorithmic_bytes_per_launch"])
    return {"floor_fetch_over_algorithmic": round(ratio, 4), "ok": ratio >= 0.98,
            "source": os.path.relpath(TRAFFIC_PROFILE, ROOT)}


def gemv_source_hash():
    """sha256 over the matvec sources with comments and whitespace removed
    (a comment edit does not change the kernel the counters measured)"""
    import hashlib
    import re
    h = hashlib.sha256()
    for rel in GEMV_SOURCES:
        with open(os.path.join(ROOT, rel)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def pmc_launches(torch, q, synth, seed):
    """The headline gate/up matvec (IQ2_K, T=1) 64 times over rotating pools and
    fresh ids, its deleted-decode floor on the same 64 launches, then the
    calibration kernels: iqk_stream_read of exactly 256 MiB (reads) and a
    256 MiB fill (writes), 8 times each."""
    gate_up = Pools(q, torch, q.IQ2_K, 2 * I, H, seed)
    values = synth.values_table(seed + 1)
    x = torch.from_numpy(synth.normal((1, H), seed + 2)).to(torch.bfloat16).cuda()
    y = torch.empty((1, K, 2 * I), dtype=torch.float32, device="cuda")
    ids = [torch.from_numpy(synth.topk_ids(1, K, E, 10_000 + i)).cuda() for i in range(64)]
    sink = torch.empty((1, K, 2 * I), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    for i in range(64):
        q.moe_gemv(gate_up.w[i % POOLS], x, ids[i], values, y=y)
    torch.cuda.synchronize()
    # the deleted-decode floor on the same launches (its HBM bytes must match the decode's)
    for i in range(64):
        q.floor_gemv(gate_up.w[i % POOLS], x, ids[i], values, sink=sink)
    torch.cuda.synchronize()
    buf = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    ssink = torch.zeros(1 << 14, dtype=torch.int32, device="cuda")
    for _ in range(8):
        q.stream_read(buf, ssink)
    for _ in range(8):
        buf.fill_(3)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_launches": 64, "gemv_bytes_per_launch_algorithmic":
                      float(np.mean([gate_up.bytes_for(a.cpu().numpy()) for a in ids])) + x.numel() * 2 + y.numel() * 4,
                      "calibration_bytes": 256 << 20}))


def sweep(ctx, fmt, Ts, seed, pools=4):
    """Decode <-> prefill crossover: for each token count T, the per-pair
    decode matvec, the fused prefill (route + plan + kernel, dequantization
    inside the MFMA GEMM) and the two-pass prefill (route + producer + GEMM)
    on the same weights and routing; one JSON line per (projection, T)."""
    import synth
    q, torch = ctx.q, ctx.torch
    grid = ctx.grid if fmt == 3 else None
    rows_out = []
    for proj, (rows, n) in (("gate_up", (2 * I, H)), ("down", (H, I))):
        slots = 1 if proj == "gate_up" else K
        pool = Pools(q, torch, fmt, rows, n, seed + (1 if proj == "gate_up" else 2), pools=pools)
        for T in Ts:
            S = 8
            ids_host = [synth.topk_ids(T, K, E, seed * 7919 + T * 31 + i) for i in range(S)]
            ids = [torch.from_numpy(a).cuda() for a in ids_host]
            x = torch.from_numpy(synth.normal((T, slots, n), seed + T)).to(torch.bfloat16).cuda()
            y = torch.zeros((T, K, rows), dtype=torch.float32, device="cuda")
            yf = torch.zeros_like(y)
            ws = torch.empty(q.prefill_fused_workspace_bytes(pool.w[0], T, K), dtype=torch.uint8, device="cuda")
            yg = torch.zeros_like(y)
            wsg = torch.empty(q.gemv_grouped_workspace_bytes(pool.w[0], T, K), dtype=torch.uint8, device="cuda")
            q.moe_gemv(pool.w[0], x, ids[0], ctx.values, grid, x_slots=slots, y=y)
            q.moe_prefill_fused(pool.w[0], x, ids[0], ctx.values, grid, x_slots=slots, workspace=ws, y=yf)
            q.moe_gemv_grouped(pool.w[0], x, ids[0], ctx.values, grid, x_slots=slots, workspace=wsg, y=yg)
            torch.cuda.synchronize()
            diff = float((yf - y).abs().max() / y.abs().max().clamp_min(1e-30))
            gdiff = float((yg - y).abs().max() / y.abs().max().clamp_min(1e-30))
            gemv_ms = timed_graph(torch, lambda i: q.moe_gemv(pool.w[i % pools], x, ids[i], ctx.values, grid,
                                                              x_slots=slots, y=y), S, 4, 1)
            grouped_ms = timed_eager(torch, lambda i: q.moe_gemv_grouped(pool.w[i % pools], x, ids[i % S], ctx.values,
                                                                         grid, x_slots=slots, workspace=wsg, y=yg),
                                     2 * S, pools)
            fused_ms = timed_eager(torch, lambda i: q.moe_prefill_fused(pool.w[i % pools], x, ids[i % S], ctx.values,
                                                                        grid, x_slots=slots, workspace=ws, y=yf),
                                   2 * S, pools)
            wsz = q.prefill_workspace_bytes(pool.w[0], T, K)
            ws2 = torch.empty(wsz, dtype=torch.uint8, device="cuda")
            two_ms = timed_eager(torch, lambda i: q.moe_prefill(pool.w[i % pools], x, ids[i % S], ctx.values, grid,
                                                                x_slots=slots, workspace=ws2, y=yf), 3, 1)
            del ws2
            distinct = float(np.mean([len(np.unique(a)) for a in ids_host]))
            times = {"gemv": gemv_ms, "grouped_gemv": grouped_ms, "fused_prefill": fused_ms,
                     "two_pass_prefill": two_ms}
            row = {"sweep": FMT_NAME[fmt], "proj": proj, "T": T, "pairs": T * K, "distinct_experts": distinct,
                   **{k + "_us": round(v * 1e3, 1) for k, v in times.items()},
                   "best": min(times, key=times.get), "fused_vs_gemv_max_rel_diff": diff,
                   "grouped_vs_gemv_max_rel_diff": gdiff}
            log(json.dumps(row))
            rows_out.append(row)
            del y, yf, yg, ws, wsg, x
        del pool
        torch.cuda.empty_cache()
    return rows_out


def _count(cells, key):
    """'passing/total' over the cells that carry the gate `key`"""
    v = [c[key] for c in cells if key in c]
    return f"{sum(bool(x) for x in v)}/{len(v)}"


def oracle_threads():
    """host threads for the all-core oracle run: the CPUs this process may
    use, at most 16 (the CPU share of one GPU on the target hosts)"""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _oracle_chunks(oracle, q, pool, experts, chunk_rows):
    """the oracle's own packing of each selected expert, in row chunks
    (units of work for the threads; each chunk is an [rows, n] tensor)"""
    rb = q.row_bytes(pool.fmt, pool.n)
    out = {}
    for e in experts:
        for r0 in range(0, pool.out, chunk_rows):
            nr = min(chunk_rows, pool.out - r0)
            a = (e * pool.out + r0) * rb
            out[(e, r0)] = (oracle.pack(pool.fmt, pool.wire[a:a + nr * rb], nr, pool.n), nr)
    return out


def _oracle_pass(oracle, pool, chunks, pairs, values, pool_exec, grid=None, w_bf16=False):
    """y (float64 [out]) for each (expert, activation row) pair through the
    oracle, one task per (pair, row chunk); pool_exec None = this thread"""
    keys = sorted(chunks)
    tasks = [(i, e, xvec, key) for i, (e, xvec) in enumerate(pairs) for key in keys if key[0] == e]

    def run(t):
        i, e, xvec, key = t
        streams, nr = chunks[key]
        return oracle.moe(pool.fmt, streams, 1, nr, pool.n, np.ascontiguousarray(xvec).reshape(1, 1, -1),
                          np.zeros((1, 1), np.int32), values, grid, w_bf16=w_bf16)[0, 0]

    parts = list(map(run, tasks)) if pool_exec is None else list(pool_exec.map(run, tasks))
    out = [np.empty(pool.out) for _ in pairs]
    for (i, e, xvec, key), yv in zip(tasks, parts):
        out[i][key[1]:key[1] + yv.size] = yv
    return out


class _WireProj:
    """one projection's stacked wire (what the oracle packs from)"""

    def __init__(self, fmt, out, n, wire):
        self.fmt, self.out, self.n, self.wire = fmt, out, n, wire


def validate_vectors(oracle, q, pool, ids, xin, y, slots, values, grid_host, pairs, w_bf16=False):
    """worst per-vector ||y - y_exact|| / ||y_exact|| over whole output
    vectors y[t, j, :] of the listed pairs (the oracle packs their experts
    from the wire itself)"""
    import concurrent.futures as cf
    chunk_rows = 256  # (a multiple of the IQ1_S_R4 four-row group)
    experts = sorted(set(int(ids[t, j]) for t, j in pairs))
    chunks = _oracle_chunks(oracle, q, pool, experts, chunk_rows)
    prs = [(int(ids[t, j]), xin[t, 0] if slots == 1 else xin[t, j]) for t, j in pairs]
    with cf.ThreadPoolExecutor(max_workers=oracle_threads()) as ex:
        refs = _oracle_pass(oracle, pool, chunks, prs, values, ex, grid_host, w_bf16)
    yv = y.cpu().numpy()
    worst = 0.0
    for (t, j), r in zip(pairs, refs):
        worst = max(worst, float(np.linalg.norm(yv[t, j] - r) / max(np.linalg.norm(r), 1e-300)))
    return worst


def sample_pairs(T, k, rng, count=8):
    """every pair of a one-token call, else `count` distinct random pairs"""
    if T == 1:
        return [(0, j) for j in range(k)]
    flat = rng.choice(T * k, size=min(count, T * k), replace=False)
    return [(int(p) // k, int(p) % k) for p in flat]


def cpu_baseline(oracle, q, synth, gate_up, down, xv, hv, ids_host, bytes_steps, values):
    """The CPU oracle on the headline workload, timed on the host: whole
    decode steps (gate/up and down matvecs of the six experts of one token),
    single-threaded and on all host threads (independent row chunks; the
    oracle's C calls release the interpreter lock), plus the prefill gate/up
    projection at 512 tokens on the pairs of a few experts, scaled to all
    256 (labelled extrapolated).  Packing by the oracle is not timed."""
    import concurrent.futures as cf
    nthreads = oracle_threads()
    chunk_rows = 256
    steps = []
    for a in ids_host[:8]:
        experts = sorted(set(int(e) for e in a.ravel()))
        steps.append((a, _oracle_chunks(oracle, q, gate_up, experts, chunk_rows),
                      _oracle_chunks(oracle, q, down, experts, chunk_rows)))

    def decode_step(i, ex):
        a, cg, cd = steps[i]
        _oracle_pass(oracle, gate_up, cg, [(int(e), xv[0, 0]) for e in a[0]], values, ex)
        _oracle_pass(oracle, down, cd, [(int(e), hv[0, j]) for j, e in enumerate(a[0])], values, ex)

    res = {}
    with cf.ThreadPoolExecutor(max_workers=nthreads) as ex:
        for label, exe, budget in (("single", None, 6.0), ("all", ex, 3.0)):
            dt, ns, nb = 0.0, 0, 0
            while ns < 1 or (dt < budget and ns < len(steps)):
                t1 = time.perf_counter()
                decode_step(ns, exe)
                dt += time.perf_counter() - t1
                nb += bytes_steps[ns]
                ns += 1
            res[label] = (nb / dt / 1e9, ns, dt)
        # prefill, gate/up at T = 512: every pair routed to the sampled experts
        T = 512
        ids = synth.topk_ids(T, K, E, 511)
        pre = {}
        for label, exe, nexp in (("single", None, 1), ("all", ex, 8)):
            experts = list(range(nexp))
            chunks = _oracle_chunks(oracle, q, gate_up, experts, chunk_rows)
            x = synth.normal((T, H), 512).astype(np.float32)
            pairs = [(int(e), x[t]) for t in range(T) for e in ids[t] if int(e) in experts]
            t1 = time.perf_counter()
            _oracle_pass(oracle, gate_up, chunks, pairs, values, exe)
            dt = time.perf_counter() - t1
            scale = (T * K) / len(pairs)
            pre[label] = {"pairs_timed": len(pairs), "experts_timed": nexp, "seconds": round(dt, 2),
                          "extrapolated_us_per_projection": round(dt * scale * 1e6, 1),
                          "extrapolated_tokens_per_s": round(T / (dt * scale), 2)}
    single, allc = res["single"], res["all"]
    return {"value": round(allc[0], 4), "unit": "GB/s", "cores": nthreads, "kind": "oracle",
            "sample": f"{allc[1]} full decode steps (T=1: gate/up and down matvecs of 6 experts each) through "
                      f"the C oracle on {nthreads} host threads in {allc[2]:.1f} s",
            "single_thread": {"value": round(single[0], 4), "unit": "GB/s", "cores": 1,
                              "sample": f"{single[1]} full decode steps in {single[2]:.1f} s"},
            "prefill_gate_up_T512": {**pre, "note": "oracle on the pairs of the timed experts, scaled by "
                                                    "pair count to all 3072 pairs (extrapolated)"},
            "host": _host_cpu()}


def write_ceiling(ctx, seed):
    """Plain streaming writes (iqk_stream_write: 16-byte non-temporal stores,
    1 KiB per wave instruction; one run per wave, and eight, the bf16
    producer's store shape) of 1.07, 2.15, 4.29 and 8.59 GB, then the bf16
    producer of each member on the two projection sizes with both writes of
    its output size, timed the same way (medians of three rounds of 50
    calls).  One JSON line per row."""
    import synth
    q, torch = ctx.q, ctx.torch
    rows = []
    buf = torch.empty(E * 2 * I * H * 2, dtype=torch.uint8, device="cuda")  # 8.59 GB: gate/up's dense bf16
    for gb_bytes in (buf.numel() // 8, buf.numel() // 4, buf.numel() // 2, buf.numel()):
        v = buf[:gb_bytes]
        for runs in (1, 8):
            ms = float(np.median([timed_eager(torch, lambda i: q.stream_write(v, 0x3F803F80, runs=runs),
                                              PREFILL_REPS, 2) for _ in range(3)]))
            rows.append({"ceiling": f"plain write, {runs} run(s) per wave", "bytes": int(gb_bytes),
                         "us": round(ms * 1e3, 1), "GBps": round(gb_bytes / (ms * 1e-3) / 1e9, 1)})
            log(json.dumps(rows[-1]))
    for fmt in (q.IQ2_K, q.IQ2_KS, q.IQ1_S_R4):
        grid = ctx.grid if fmt == q.IQ1_S_R4 else None
        for proj, (out, n) in (("gate_up", (2 * I, H)), ("down", (H, I))):
            wire = synth.wire(fmt, E * out, n, seed + fmt)
            w = q.Weights(fmt, E, out, n, torch.from_numpy(q.pack_relayout(fmt, wire, E * out, n)).cuda())
            dv = buf[:E * out * n * 2].view(torch.bfloat16).view(E * out, n)
            ms = float(np.median([timed_eager(torch, lambda i: q.dequant(w, ctx.values, grid, torch.bfloat16, out=dv),
                                              PREFILL_REPS, 2) for _ in range(3)]))
            wms = float(np.median([timed_eager(torch, lambda i: q.stream_write(dv, 0x3F803F80), PREFILL_REPS, 2)
                                   for _ in range(3)]))
            w8ms = float(np.median([timed_eager(torch, lambda i: q.stream_write(dv, 0x3F803F80, runs=8),
                                                PREFILL_REPS, 2) for _ in range(3)]))
            wb = E * out * n * 2
            rb = E * out * q.row_bytes(fmt, n)
            rows.append({"producer": f"{FMT_NAME[fmt]} {proj} bf16", "us": round(ms * 1e3, 1),
                         "bytes": int(wb + rb), "GBps": round((wb + rb) / (ms * 1e-3) / 1e9, 1),
                         "write_ceiling_us": round(wms * 1e3, 1),
                         "vs_write_ceiling": round(wms / ms, 3),
                         "same_shape_write_us": round(w8ms * 1e3, 1),
                         "vs_same_shape_write": round(w8ms / ms, 3)})
            log(json.dumps(rows[-1]))
            del w
            torch.cuda.empty_cache()
    return rows


def main():
    args = _parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "bench.py runs on exactly one GPU; multi-GPU runs are not provided "
                                   "(the expert-parallel sharding is described, not built)"}))
        sys.exit(2)

    import torch
    import dequant_iqk_moe_amd as q
    import synth
    import oracle

    torch.cuda.set_device(0)
    if args.mode == "pmc":
        pmc_launches(torch, q, synth, args.seed)
        return
    if args.mode == "ceiling":
        rows = write_ceiling(Ctx(q, torch, args.seed), 800)
        print(json.dumps({"ceiling_rows": rows}), flush=True)
        return
    if args.mode == "sweep":
        ctx = Ctx(q, torch, args.seed)
        rows = []
        for fmt in (q.IQ2_K, q.IQ2_KS, q.IQ1_S_R4):
            rows += sweep(ctx, fmt, (1, 2, 4, 8, 16, 32, 64, 128, 256, 512), 900 + fmt)
        best = {}
        for r in rows:
            best.setdefault(f"{r['sweep']} {r['proj']}", []).append((r["T"], r["best"]))
        print(json.dumps({"sweep_rows": len(rows), "best_path_by_T": best}), flush=True)
        return
    T = 1
    # steps per captured graph: the largest divisor of K up to 64, so exactly K steps are timed
    S = max(d for d in range(1, 65) if args.steps % d == 0)
    reps = args.steps // S
    warm = max(1, -(-args.warmup // S))
    t0 = time.time()
    ctx = Ctx(q, torch, args.seed)
    gate_up = Pools(q, torch, q.IQ2_K, 2 * I, H, args.seed)
    down = Pools(q, torch, q.IQ2_K, H, I, args.seed + 100)
    values = ctx.values
    ids_host = [synth.topk_ids(T, K, E, 10_000 + i) for i in range(S)]
    ids_dev = [torch.from_numpy(a).cuda() for a in ids_host]
    x = torch.from_numpy(synth.normal((T, H), args.seed + 2)).to(torch.bfloat16).cuda()
    h = torch.from_numpy(synth.normal((T, K, I), args.seed + 3)).to(torch.bfloat16).cuda()
    y1 = torch.empty((T, K, 2 * I), dtype=torch.float32, device="cuda")
    y2 = torch.empty((T, K, H), dtype=torch.float32, device="cuda")
    setup_s = time.time() - t0

    # validation on the exact timed inputs before any timing (sampled rows)
    q.moe_gemv(gate_up.w[0], x, ids_dev[0], values, y=y1)
    q.moe_gemv(down.w[0], h, ids_dev[0], values, x_slots=K, y=y2)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    xv = x.float().cpu().numpy().reshape(T, 1, H)
    hv = h.float().cpu().numpy()
    worst = max(validate_vectors(oracle, q, gate_up, ids_host[0], xv, y1, 1, values, None, sample_pairs(T, K, rng)),
                validate_vectors(oracle, q, down, ids_host[0], hv, y2, K, values, None, sample_pairs(T, K, rng)))
    if worst > 1e-3:
        print(json.dumps({"error": f"validation failed: worst per-vector error {worst:.3e}"}))
        sys.exit(1)

    def step(i):
        p = i % POOLS
        q.moe_gemv(gate_up.w[p], x, ids_dev[i], values, y=y1)
        q.moe_gemv(down.w[p], h, ids_dev[i], values, x_slots=K, y=y2)

    # warm-up: `warm` graph replays, then the same untimed clock ramp every
    # other cell gets (the GPU lowers its clocks while the host validates)
    head_info = {}
    ms_step = timed_graph(torch, step, S, reps, warm, info=head_info)
    bytes_steps = [gate_up.bytes_for(a) + down.bytes_for(a) + x.numel() * 2 + y1.numel() * 4 + h.numel() * 2
                   + y2.numel() * 4 for a in ids_host]
    bytes_per_step = float(np.mean(bytes_steps))
    gbs = bytes_per_step / (ms_step * 1e-3) / 1e9
    log(f"headline step: {ms_step * 1e3:.2f} us, {gbs:.1f} GB/s")

    # dominant kernel: the gate/up matvec alone, its floor and a same-size streaming read
    def gu(i):
        q.moe_gemv(gate_up.w[i % POOLS], x, ids_dev[i], values, y=y1)

    ms_gu = timed_graph(torch, gu, S, reps, warm)
    gu_bytes = float(np.mean([gate_up.bytes_for(a) + x.numel() * 2 + y1.numel() * 4 for a in ids_host]))
    gu_gbs = gu_bytes / (ms_gu * 1e-3) / 1e9
    sink = torch.empty((T, K, 2 * I), dtype=torch.int32, device="cuda")

    def gu_floor(i):
        q.floor_gemv(gate_up.w[i % POOLS], x, ids_dev[i], values, sink=sink)

    ms_floor = timed_graph(torch, gu_floor, S, reps, warm)
    ms_stream = ctx.stream_ms(gu_bytes, S, reps, warm)

    cells = []
    if args.cells == "all":
        Sc, rc, wc = 32, 8, 2
        cells.append(layer_cell(ctx, gate_up, down, x, Sc, rc, wc, 61))
        cells.append(decode_cell(ctx, gate_up, 1, "gate_up", Sc, rc, wc, 21))
        cells.append(decode_cell(ctx, down, 1, "down", Sc, rc, wc, 22))
        for fmt, Ts, sd in ((q.IQ2_KS, (1, 8), 3), (q.IQ1_S_R4, (1,), 4)):
            pg = Pools(q, torch, fmt, 2 * I, H, 100 + sd)
            pd = Pools(q, torch, fmt, H, I, 200 + sd)
            for Tt in Ts:
                cells.append(decode_cell(ctx, pg, Tt, "gate_up", Sc, rc, wc, 30 + sd + Tt))
                cells.append(decode_cell(ctx, pd, Tt, "down", Sc, rc, wc, 40 + sd + Tt))
            del pg, pd
            torch.cuda.empty_cache()
        # the single-matrix case: IQ2_KS [256, 512], fp32 activation, E = 1, k = 1
        w1 = q.Weights.from_wire(q.IQ2_KS, 1, 256, 512, synth.wire(q.IQ2_KS, 256, 512, 1))
        x1 = torch.from_numpy(synth.normal((1, 512), 1)).cuda()
        id1 = torch.zeros((1, 1), dtype=torch.int32, device="cuda")
        y1s = torch.empty((1, 1, 256), dtype=torch.float32, device="cuda")
        ms1 = timed_graph(torch, lambda i: q.moe_gemv(w1, x1, id1, values, y=y1s), Sc, rc, wc)
        b1 = 256 * q.row_bytes(q.IQ2_KS, 512) + 512 * 4 + 256 * 4
        cells.append({"cell": "IQ2_KS single [256,512] fp32 x", "kind": "decode", "us": round(ms1 * 1e3, 3),
                      "bytes": b1, "GBps": round(b1 / (ms1 * 1e-3) / 1e9, 2)})
    if args.cells in ("all", "prefill"):
        ctx.sbuf = None
        torch.cuda.empty_cache()
        for fmt in (q.IQ2_K, q.IQ2_KS, q.IQ1_S_R4):
            cells.extend(prefill_cells(ctx, fmt, 500 + fmt))
        cells.append(prefill_layer_cell(ctx, 600))
    for c in cells:
        log(json.dumps(c))

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(oracle, q, synth, gate_up, down, xv, hv, ids_host, bytes_steps, values)

    result = {
        "metric": "routed-expert decode GB/s and ratio to HBM floor per format/projection",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": reps * S,
        "warmup": head_info["untimed_replays"] * S,
        "ms_per_step": round(ms_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8-decode/fp32-acc",
        "data": "synthetic",
        "config": {"workload": "IQ2_K routed MoE decode, T=1, top-6 of 256 experts, gate/up [2048,4096] "
                               "(fused) + down [4096,2048], bf16 activations",
                   "experts": E, "top_k": K, "tokens": T, "hidden": H, "intermediate": I,
                   "bytes_per_step": int(bytes_per_step), "weight_pools": POOLS, "graph_steps": S},
        "fraction_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(T / (ms_step * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(gu_gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gu_gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(), "traffic_unit": "bytes/launch",
                     "kernel": "gemv_kernel<IQ2_K, 4096, bf16> (gate/up)",
                     "bytes_per_launch": int(gu_bytes), "us_per_launch": round(ms_gu * 1e3, 3)},
        "ratio_to_own_floor": round(ms_gu / ms_floor, 4),
        "floor_us_per_launch": round(ms_floor * 1e3, 3),
        "stream_read_us_same_bytes": round(ms_stream * 1e3, 3),
        "validation_worst_err": worst,
        "setup_s": round(setup_s, 1),
        "warmup_detail": {"requested_steps": args.warmup, "graph_replays_requested": warm,
                          "clock_ramp_s": CLOCK_RAMP_S, "untimed_steps_run": head_info["untimed_replays"] * S},
        "cells_passing_ratio_bar": _count(cells, "ratio_ok"),
        "cells_passing_floor_band": _count(cells, "band_ok"),
        "deleted_load_check": deleted_load_check(),
        "cells": cells,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
