"""GPU parity of the HIP path against the CPU oracle (run on an MI355X).

Inputs come from ``synth`` (seeded); expected values come from ``oracle``
only.  Bars ("mlx-iqk" description and the accuracy targets of this path):
dequantization bit-exact (float32, and the f16 / bf16 casts after RNE),
relayout byte-exact (CPU tests), matvec rel. err <= 1e-3 per output vector,
bf16-weight GEMM <= 2e-2 against the float32-weight product, routing
bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import dequant_iqk_moe_amd as q
from gpu_common import TOL_BF16, TOL_GEMV, announce, bf16_round, rel_err_per_vector, to_dev

pytestmark = pytest.mark.gpu

KS, K, R4 = 1, 2, 3
DT = {oracle.F32: torch.float32, oracle.F16: torch.float16, oracle.BF16: torch.bfloat16}


def _weights(fmt, E, out, n, seed):
    wire = synth.wire(fmt, E * out, n, seed)
    w = q.Weights.from_wire(fmt, E, out, n, wire)
    return wire, w, oracle.pack(fmt, wire, E * out, n)


def _bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.float32:
        return t.cpu().view(torch.int32).numpy().view(np.uint32)
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


# ---------------------------------------------------------------------------
# dequantization: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", [oracle.F32, oracle.F16, oracle.BF16])
@pytest.mark.parametrize("fmt,E,out,n,row0,nrows", [
    (KS, 3, 40, 512, 0, None), (KS, 2, 9, 4096, 5, 11),
    (K, 3, 40, 768, 0, None), (K, 2, 33, 2048, 17, 31),
    (R4, 2, 12, 96, 0, None), (R4, 3, 8, 4096, 3, 17),
])
def test_dequant_bit_exact(fmt, E, out, n, row0, nrows, dtype):
    announce(f"dequant fmt={fmt} E={E} out={out} n={n} rows=({row0},{nrows}) dtype={dtype}")
    _, w, s = _weights(fmt, E, out, n, 100 + fmt + n)
    values = synth.values_table(3)
    grid = synth.ternary_grid(4)
    nr = E * out - row0 if nrows is None else nrows
    got = q.dequant(w, values, to_dev(grid), DT[dtype], row0=row0, nrows=nr)
    torch.cuda.synchronize()
    exp = oracle.dequant(fmt, s, E * out, n, values, grid, dtype, r0=row0, nr=nr)
    exp_bits = exp.view(np.uint32) if dtype == oracle.F32 else exp
    assert np.array_equal(_bits(got).reshape(exp_bits.shape), exp_bits)


def test_dequant_general_float_tables_and_edge_scales():
    # non-integer tables (rounding of both multiplies matters), tiny table
    # values (float32 subnormal products), zero scales (signed zeros)
    rng = np.random.default_rng(5)
    fmt, E, out, n = KS, 2, 16, 512
    wire = synth.wire(fmt, E * out, n, 55, sigma=0.37)
    rb = oracle.row_bytes(fmt, n)
    wire.reshape(E * out, rb)[0, 0:2] = [0x01, 0x00]     # fp16 subnormal row scale
    wire.reshape(E * out, rb)[1, 0:2] = [0x00, 0x80]     # -0.0 row scale
    w = q.Weights.from_wire(fmt, E, out, n, wire)
    s = oracle.pack(fmt, wire, E * out, n)
    for values in ((rng.standard_normal(8) * 3).astype(np.float32),
                   np.array([1e-39, -3e-40, 2e-38, 7e-45, -1e-44, 5e-39, 0.0, -0.0], np.float32)):
        for dtype in (oracle.F32, oracle.F16, oracle.BF16):
            announce(f"dequant edge values={values[:2]} dtype={dtype}")
            got = _bits(q.dequant(w, values, None, DT[dtype]))
            exp = oracle.dequant(fmt, s, E * out, n, values, None, dtype)
            exp = exp.view(np.uint32) if dtype == oracle.F32 else exp
            assert np.array_equal(got.reshape(exp.shape), exp)


# ---------------------------------------------------------------------------
# decode matvec: rel. err <= 1e-3 per output vector
# ---------------------------------------------------------------------------

def _gemv_case(fmt, n, out, T, k, E, x_dtype, x_slots, seed):
    _, w, s = _weights(fmt, E, out, n, seed)
    values = synth.values_table(seed + 1)
    grid = synth.ternary_grid(seed + 2)
    ids = synth.topk_ids(T, k, E, seed + 3)
    x = synth.normal((T, x_slots, n), seed + 4)
    if x_dtype == torch.bfloat16:
        x = bf16_round(x)
    y = q.moe_gemv(w, to_dev(x, x_dtype), to_dev(ids), values, to_dev(grid), x_slots=x_slots)
    torch.cuda.synchronize()
    ref = oracle.moe(fmt, s, E, out, n, x, ids, values, grid, x_slots=x_slots)
    return y.cpu().numpy(), ref


@pytest.mark.parametrize("x_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("fmt", [KS, K, R4])
@pytest.mark.parametrize("n,out,T,k,E,x_slots", [
    (4096, 72, 3, 4, 8, 1),     # ragged last row block
    (2048, 72, 3, 4, 8, 4),     # per-pair input (down)
    (512, 72, 2, 3, 5, 1),
    (2048, 4100, 1, 2, 3, 1),   # several groups per wave, ragged tail of 4 rows
    (512, 8, 300, 6, 40, 6),    # blocks span four pairs, four activation rows each
    (4096, 12, 50, 6, 20, 1),   # blocks span pairs of two tokens
    (2048, 6, 40, 5, 10, 5),    # two-row groups per pair, ragged, per-pair input
])
def test_gemv_parity(fmt, n, out, T, k, E, x_slots, x_dtype):
    announce(f"gemv fmt={fmt} n={n} out={out} T={T} k={k} E={E} slots={x_slots} x={x_dtype}")
    y, ref = _gemv_case(fmt, n, out, T, k, E, x_dtype, x_slots, 200 + fmt + n // 256 + out)
    err = rel_err_per_vector(y, ref)
    assert np.all(err <= TOL_GEMV), err.max()


def test_gemv_deterministic_and_order_free():
    fmt, n, out, E = K, 4096, 64, 16
    _, w, s = _weights(fmt, E, out, n, 301)
    values = synth.values_table(302)
    x = bf16_round(synth.normal((4, 1, n), 303))
    ids = synth.topk_ids(4, 6, E, 304)
    xd, idd = to_dev(x, torch.bfloat16), to_dev(ids)
    announce("gemv determinism")
    a = q.moe_gemv(w, xd, idd, values).cpu().numpy()
    b = q.moe_gemv(w, xd, idd, values).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # permuting the slots of each token permutes the outputs bit for bit
    perm = np.array([3, 0, 5, 1, 4, 2])
    c = q.moe_gemv(w, xd, to_dev(np.ascontiguousarray(ids[:, perm])), values).cpu().numpy()
    assert np.array_equal(c.view(np.uint32), a[:, perm].view(np.uint32))
    # duplicated tokens give identical rows
    x2 = np.concatenate([x[:1], x[:1]])
    ids2 = np.concatenate([ids[:1], ids[:1]])
    d = q.moe_gemv(w, to_dev(x2, torch.bfloat16), to_dev(ids2), values).cpu().numpy()
    assert np.array_equal(d[0].view(np.uint32), d[1].view(np.uint32))


@pytest.mark.parametrize("fmt", [KS, K, R4])
def test_gemv_one_hot_reads_one_column(fmt):
    n, out, E = 2048, 64, 4
    _, w, s = _weights(fmt, E, out, n, 400 + fmt)
    values = synth.values_table(401)
    grid = synth.ternary_grid(402)
    W = oracle.dequant(fmt, s, E * out, n, values, grid).reshape(E, out, n)
    cols = [0, 1, 63, 64, 1000, 2047]
    x = np.zeros((len(cols), 1, n), np.float32)
    for i, c in enumerate(cols):
        x[i, 0, c] = 1.0
    ids = np.full((len(cols), 1), 2, np.int32)
    announce(f"gemv one-hot fmt={fmt}")
    y = q.moe_gemv(w, to_dev(x, torch.bfloat16), to_dev(ids), values, to_dev(grid)).cpu().numpy()
    for i, c in enumerate(cols):
        np.testing.assert_allclose(y[i, 0], W[2, :, c], rtol=1e-6, atol=1e-30)


def test_gemv_invalid_ids_give_nan_rows():
    fmt, n, out, E = KS, 512, 40, 3
    _, w, s = _weights(fmt, E, out, n, 500)
    values = synth.values_table(501)
    ids = np.array([[0, 7, -1, 2]], np.int32)
    x = bf16_round(synth.normal((1, 1, n), 502))
    announce("gemv invalid ids")
    y = q.moe_gemv(w, to_dev(x, torch.bfloat16), to_dev(ids), values).cpu().numpy()
    assert np.all(np.isnan(y[0, 1])) and np.all(np.isnan(y[0, 2]))
    ref = oracle.moe(fmt, s, E, out, n, x, ids, values)
    assert np.all(rel_err_per_vector(y[0, [0, 3]], ref[0, [0, 3]]) <= TOL_GEMV)


@pytest.mark.parametrize("fmt", [KS, R4])
@pytest.mark.parametrize("n", [2048, 4096])
def test_gemv_invalid_ids_wide_rows(fmt, n):
    # the per-row scale of these widths comes through a scalar load from the
    # expert's plane (expert 0's for an invalid id, clamped rows past the
    # last): invalid pairs still read NaN and the valid ones stay exact
    out, E = (68 if fmt == R4 else 70), 3  # IQ2_KS: a ragged last row group
    _, w, s = _weights(fmt, E, out, n, 520 + n // 1024 + fmt)
    values = synth.values_table(521)
    grid = synth.ternary_grid(522)
    ids = np.array([[0, 7, -1, 2], [2, 1, 5, 0]], np.int32)
    x = bf16_round(synth.normal((2, 1, n), 523))
    announce(f"gemv invalid ids fmt={fmt} n={n}")
    y = q.moe_gemv(w, to_dev(x, torch.bfloat16), to_dev(ids), values, to_dev(grid)).cpu().numpy()
    bad = (ids < 0) | (ids >= E)
    assert np.all(np.isnan(y[bad]))
    ref = oracle.moe(fmt, s, E, out, n, x, np.where(bad, 0, ids).astype(np.int32), values, grid)
    assert np.all(rel_err_per_vector(y[~bad], ref[~bad]) <= TOL_GEMV)


def test_gemv_invalid_ids_inside_multi_pair_blocks():
    # out = 8 rows at n = 512 is one reduction group per pair, so every
    # workgroup spans several pairs; invalid ids must only blank their own
    fmt, n, out, E, T, k = K, 512, 8, 12, 64, 6
    _, w, s = _weights(fmt, E, out, n, 510)
    values = synth.values_table(511)
    ids = synth.topk_ids(T, k, E, 512)
    rng = np.random.default_rng(513)
    bad = rng.random(ids.shape) < 0.15
    ids = np.where(bad, np.where(rng.random(ids.shape) < 0.5, -3, E + 4), ids).astype(np.int32)
    x = bf16_round(synth.normal((T, k, n), 514))
    announce("gemv invalid ids in multi-pair blocks")
    y = q.moe_gemv(w, to_dev(x, torch.bfloat16), to_dev(ids), values, x_slots=k).cpu().numpy()
    assert np.all(np.isnan(y[bad]))
    ref = oracle.moe(fmt, s, E, out, n, x, ids, values, x_slots=k)
    assert np.all(rel_err_per_vector(y[~bad], ref[~bad]) <= TOL_GEMV)


def test_gemv_activation_outliers_and_zeros():
    # per-64 block scaling keeps accuracy when one channel is 1000x larger
    fmt, n, out, E = K, 4096, 32, 2
    _, w, s = _weights(fmt, E, out, n, 600)
    values = synth.values_table(601)
    x = synth.normal((3, 1, n), 602)
    x[0, 0, 17] = 3000.0
    x[1, 0, :] = 0.0
    x[1, 0, 4095] = 1e-30
    x[2, 0, 64:128] = 0.0
    ids = np.array([[1], [0], [1]], np.int32)
    announce("gemv outliers")
    y = q.moe_gemv(w, to_dev(x, torch.float32), to_dev(ids), values).cpu().numpy()
    ref = oracle.moe(fmt, s, E, out, n, x, ids, values)
    assert np.all(rel_err_per_vector(y, ref) <= TOL_GEMV)


# ---------------------------------------------------------------------------
# routing gather: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,k,E", [(1, 6, 256), (8, 6, 256), (512, 6, 256), (37, 3, 5), (3000, 8, 1000),
                                   (700, 8, 3000)])   # more than 1024 experts: one wave ranks
def test_route_bit_exact(T, k, E):
    ids = synth.topk_ids(T, k, E, 700 + T)
    announce(f"route T={T} k={k} E={E}")
    counts, offsets, perm = q.route(to_dev(ids), E)
    c0, o0, p0, bad = oracle.route(ids, E)
    assert np.array_equal(counts.cpu().numpy(), c0)
    assert np.array_equal(offsets.cpu().numpy(), o0)
    assert np.array_equal(perm.cpu().numpy(), p0)
    # sorted ids with the caller's sort flag: the identity permutation
    # (the flag's full contract is in test_gpu_contract.py)
    s_ids = np.sort(ids.ravel()).reshape(ids.shape).astype(np.int32)
    _, _, ps = q.route(to_dev(s_ids), E, sorted=True)
    assert np.array_equal(ps.cpu().numpy(), np.arange(ids.size))


def test_route_drops_invalid_ids():
    ids = np.array([[3, -1, 0], [9, 3, 1]], np.int32)
    counts, offsets, perm = q.route(to_dev(ids), 4)
    c0, o0, p0, bad = oracle.route(ids, 4)
    assert np.array_equal(counts.cpu().numpy(), c0)
    assert np.array_equal(offsets.cpu().numpy(), o0)
    got = perm.cpu().numpy()
    assert np.array_equal(got[: p0.size], p0) and np.all(got[p0.size:] == -1)


def test_route_invalid_ids_across_staging_chunks():
    """4400 pairs (ids are staged 4096 at a time), invalid ids on both sides
    of the chunk boundary"""
    T, k, E = 1100, 4, 37
    ids = synth.topk_ids(T, k, E, 771)
    flat = ids.reshape(-1)
    flat[[5, 4095, 4096, 4097, 4399]] = [-1, E, -7, E + 100, -1]
    announce("route: invalid ids across staging chunks")
    counts, offsets, perm = q.route(to_dev(ids), E)
    c0, o0, p0, bad = oracle.route(ids, E)
    assert np.array_equal(counts.cpu().numpy(), c0)
    assert np.array_equal(offsets.cpu().numpy(), o0)
    got = perm.cpu().numpy()
    assert np.array_equal(got[: p0.size], p0) and np.all(got[p0.size:] == -1)


# ---------------------------------------------------------------------------
# grouped GEMM and prefill
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt,E,out,n,T,k,x_slots", [(K, 8, 64, 256, 40, 3, 1), (K, 5, 272, 512, 77, 2, 2),
                                                     (R4, 3, 48, 192, 1, 1, 1)])
def test_grouped_gemm_matches_bf16_weight_product(fmt, E, out, n, T, k, x_slots):
    _, _, s = _weights(fmt, E, out, n, 800 + E)
    values = synth.values_table(801)
    grid = synth.ternary_grid(805)
    Wb = oracle.dequant(fmt, s, E * out, n, values, grid, oracle.BF16).reshape(E, out, n)
    Wd = torch.from_numpy(Wb.view(np.int16)).view(torch.bfloat16).cuda()
    x = bf16_round(synth.normal((T, x_slots, n), 802))
    ids = synth.topk_ids(T, k, E, 803)
    announce(f"grouped gemm E={E} out={out} n={n} T={T} k={k}")
    counts, offsets, perm = q.route(to_dev(ids), E)
    y = q.grouped_gemm(Wd, to_dev(x, torch.bfloat16), T, k, offsets, perm, x_slots=x_slots).cpu().numpy()
    ref = oracle.moe(fmt, s, E, out, n, x, ids, values, grid, x_slots=x_slots, w_bf16=True)
    assert np.all(rel_err_per_vector(y, ref) <= TOL_GEMV)


@pytest.mark.parametrize("fmt", [KS, K, R4])
def test_prefill_matches_oracle(fmt):
    E, out, n, T, k = 16, 96, 512, 64, 6
    _, w, s = _weights(fmt, E, out, n, 900 + fmt)
    values = synth.values_table(901)
    grid = synth.ternary_grid(902)
    x = bf16_round(synth.normal((T, 1, n), 903))
    ids = synth.topk_ids(T, k, E, 904)
    announce(f"prefill fmt={fmt}")
    y = q.moe_prefill(w, to_dev(x, torch.bfloat16), to_dev(ids), values, to_dev(grid)).cpu().numpy()
    ref = oracle.moe(fmt, s, E, out, n, x, ids, values, grid)
    assert np.all(rel_err_per_vector(y, ref) <= TOL_BF16)
    ref_b = oracle.moe(fmt, s, E, out, n, x, ids, values, grid, w_bf16=True)
    assert np.all(rel_err_per_vector(y, ref_b) <= TOL_GEMV)


# ---------------------------------------------------------------------------
# measurement kernels run and touch every output
# ---------------------------------------------------------------------------

def test_floor_and_stream_kernels_run():
    fmt, n, out, E = K, 4096, 64, 4
    _, w, s = _weights(fmt, E, out, n, 950)
    values = synth.values_table(951)
    ids = synth.topk_ids(2, 3, E, 952)
    x = to_dev(bf16_round(synth.normal((2, 1, n), 953)), torch.bfloat16)
    announce("floor kernels")
    sink = torch.full((2, 3, out), -7, dtype=torch.int32, device="cuda")
    q.floor_gemv(w, x, to_dev(ids), values, sink=sink)
    o = torch.full((E * out, n), -7, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    q.floor_dequant(w, torch.bfloat16, out=o)
    buf = torch.ones(1 << 20, dtype=torch.int32, device="cuda")
    sk = torch.zeros(1024, dtype=torch.int32, device="cuda")
    q.stream_read(buf, sk)
    torch.cuda.synchronize()
    assert not torch.any(sink == -7).item()


@pytest.mark.parametrize("runs", [1, 8, 16])
def test_stream_write_fills_exactly_its_buffer(runs):
    """every 16-byte word of the buffer written, none past it, also for a
    size that ends inside a workgroup's span"""
    announce(f"stream write runs={runs}")
    words = 256 * runs * 5 + 4 * 37  # 16-byte words: five full workgroups and a ragged tail
    guard = 256
    buf = torch.zeros((words + guard) * 4, dtype=torch.int32, device="cuda")
    q.stream_write(buf[:words * 4], 0x3F803F80, runs=runs)
    torch.cuda.synchronize()
    h = buf.cpu().numpy().view(np.uint32)
    assert np.all(h[:words * 4] == 0x3F803F80)
    assert np.all(h[words * 4:] == 0)
