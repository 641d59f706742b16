"""GPU tests of the call contract beyond the default inputs (run on an MI355X).

* the caller's sort flag ("mlx-iqk" package description, "Surface": pairs
  sorted by expert read each expert once): sorted=1 on ids that are
  non-decreasing gives the same bits as sorted=0 on every routed call, and
  sorted=1 on ids that are not in order still gives the stable sort;
* one rule for invalid ids on every routed path: NaN output rows, the other
  rows as the oracle gives them, whatever path the dispatcher takes;
* value tables of the form m_i * 2^e with e != 0 (the decode matvec's
  scaled int8 table) and an IQ1_S_R4 grid holding other int8 values than
  -1, 0, +1 (the float32 producer and the matvecs compute them; the paths
  that rely on a ternary grid return NaN).

Expected values come from ``oracle`` only; inputs from ``synth``.
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


def _weights(fmt, E, out, n, seed):
    wire = synth.wire(fmt, E * out, n, seed)
    return q.Weights.from_wire(fmt, E, out, n, wire), oracle.pack(fmt, wire, E * out, n)


def _bits(y: torch.Tensor) -> np.ndarray:
    return y.cpu().numpy().view(np.uint32)


# ---------------------------------------------------------------------------
# the caller's sort flag
# ---------------------------------------------------------------------------

def _sorted_ids(P, E, seed, n_neg=0, n_big=0):
    """[P, 1] non-decreasing ids: n_neg ids below zero first, n_big ids >= E last"""
    rng = np.random.default_rng(seed)
    mid = np.sort(rng.integers(0, E, size=P - n_neg - n_big))
    ids = np.concatenate([np.sort(rng.integers(-5, 0, size=n_neg)), mid, np.sort(rng.integers(E, E + 9, size=n_big))])
    return ids.astype(np.int32).reshape(P, 1)


@pytest.mark.parametrize("P,E,n_neg,n_big", [(96, 16, 0, 0), (700, 40, 3, 5), (5000, 300, 0, 2)])
def test_route_sorted_flag_identity(P, E, n_neg, n_big):
    ids = _sorted_ids(P, E, 1000 + P, n_neg, n_big)
    announce(f"route sorted=1 P={P} E={E} invalid={n_neg}+{n_big}")
    c1, o1, p1 = q.route(to_dev(ids), E, sorted=True)
    c0, o0, p0 = q.route(to_dev(ids), E, sorted=False)
    ce, oe, pe, bad = oracle.route(ids, E)
    assert bad == n_neg + n_big
    for a, b, e in ((c1, c0, ce), (o1, o0, oe)):
        assert np.array_equal(a.cpu().numpy(), e) and np.array_equal(b.cpu().numpy(), e)
    got1, got0 = p1.cpu().numpy(), p0.cpu().numpy()
    assert np.array_equal(got1, got0)
    assert np.array_equal(got1[: pe.size], pe) and np.all(got1[pe.size:] == -1)
    # the stable sort of sorted ids is the identity on the valid pairs
    assert np.array_equal(pe, np.arange(n_neg, P - n_big))


def test_route_sorted_flag_on_unsorted_ids_still_sorts():
    T, k, E = 300, 6, 64
    ids = synth.topk_ids(T, k, E, 1101)
    announce("route sorted=1 on ids out of order")
    _, _, p1 = q.route(to_dev(ids), E, sorted=True)
    _, _, pe, _ = oracle.route(ids, E)
    assert np.array_equal(p1.cpu().numpy(), pe)


@pytest.mark.parametrize("fmt", [KS, K, R4])
def test_routed_calls_with_sorted_flag(fmt):
    """moe_gemv_grouped, moe_prefill and moe_prefill_fused with sorted=1 on
    pre-sorted pairs: the same bits as sorted=0, and the oracle's product"""
    E, out, n, P = 24, 64, 512, 120
    w, s = _weights(fmt, E, out, n, 1200 + fmt)
    values = synth.values_table(1201)
    grid = synth.ternary_grid(1202)
    ids = _sorted_ids(P, E, 1203)
    x = bf16_round(synth.normal((P, 1, n), 1204))
    xd, idd, gd = to_dev(x, torch.bfloat16), to_dev(ids), to_dev(grid)
    ref = oracle.moe(fmt, s, E, out, n, x, ids, values, grid)
    ref_b = oracle.moe(fmt, s, E, out, n, x, ids, values, grid, w_bf16=True)
    for name, call, bars in (
            ("grouped", q.moe_gemv_grouped, ((ref, TOL_GEMV),)),
            ("prefill", q.moe_prefill, ((ref, TOL_BF16), (ref_b, TOL_GEMV))),
            ("fused", q.moe_prefill_fused, ((ref, TOL_BF16), (ref_b, TOL_GEMV)))):
        announce(f"sorted flag fmt={fmt} {name}")
        y1 = call(w, xd, idd, values, gd, sorted=True)
        y0 = call(w, xd, idd, values, gd, sorted=False)
        torch.cuda.synchronize()
        assert np.array_equal(_bits(y1), _bits(y0)), name
        for r, tol in bars:
            assert np.all(rel_err_per_vector(y1.cpu().numpy(), r) <= tol), name


# ---------------------------------------------------------------------------
# invalid ids: NaN rows on every path
# ---------------------------------------------------------------------------

def _ids_with_invalid(T, k, E, seed):
    ids = synth.topk_ids(T, k, E, seed)
    rng = np.random.default_rng(seed + 1)
    bad = rng.random(ids.shape) < 0.1
    bad[0, 0] = True
    ids = np.where(bad, np.where(rng.random(ids.shape) < 0.5, -2, E + 3), ids).astype(np.int32)
    return ids, bad


@pytest.mark.parametrize("fmt", [K, R4])
def test_invalid_ids_nan_rows_on_every_path(fmt):
    E, out, n, T, k = 32, 48, 4096, 40, 6
    w, s = _weights(fmt, E, out, n, 1300 + fmt)
    values = synth.values_table(1301)
    grid = synth.ternary_grid(1302)
    ids, bad = _ids_with_invalid(T, k, E, 1303)
    x = bf16_round(synth.normal((T, 1, n), 1305))
    xd, idd, gd = to_dev(x, torch.bfloat16), to_dev(ids), to_dev(grid)
    ref = oracle.moe(fmt, s, E, out, n, x, ids, values, grid)
    assert np.all(np.isnan(ref[bad]))
    for name, call, tol in (("gemv", q.moe_gemv, TOL_GEMV), ("grouped", q.moe_gemv_grouped, TOL_GEMV),
                            ("prefill", q.moe_prefill, TOL_BF16), ("fused", q.moe_prefill_fused, TOL_BF16)):
        announce(f"invalid ids fmt={fmt} {name}")
        y = call(w, xd, idd, values, gd).cpu().numpy()
        assert np.all(np.isnan(y[bad])), name
        assert np.all(rel_err_per_vector(y[~bad], ref[~bad]) <= tol), name
    # the dispatcher: the same rule whichever path T selects
    for Tt in (1, 8, T):
        announce(f"invalid ids fmt={fmt} auto T={Tt}")
        y, path = q.moe_auto(w, xd[:Tt], idd[:Tt], values, gd)
        yv = y.cpu().numpy()
        assert np.all(np.isnan(yv[bad[:Tt]])), path
        tol = TOL_BF16 if path == "fused_prefill" else TOL_GEMV
        assert np.all(rel_err_per_vector(yv[~bad[:Tt]], ref[:Tt][~bad[:Tt]]) <= tol), path


# ---------------------------------------------------------------------------
# value tables m_i * 2^e with e != 0
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("e", [-1, -3])
@pytest.mark.parametrize("fmt", [KS, K])
def test_scaled_int8_tables(fmt, e):
    E, out, n, T, k = 12, 40, 2048, 6, 4
    w, s = _weights(fmt, E, out, n, 1400 + fmt)
    values = synth.values_table(1401 - e) * np.float32(2.0 ** e)   # integers times 2^e: exact
    assert np.all(values * np.float32(2.0 ** -e) == np.round(values * np.float32(2.0 ** -e)))
    ids = synth.topk_ids(T, k, E, 1402)
    x = synth.normal((T, 1, n), 1403)
    ref = oracle.moe(fmt, s, E, out, n, x, ids, values)
    for x_dtype in (torch.float32, torch.bfloat16):
        xx = bf16_round(x) if x_dtype == torch.bfloat16 else x
        r = ref if x_dtype == torch.float32 else oracle.moe(fmt, s, E, out, n, xx, ids, values)
        xd = to_dev(xx, x_dtype)
        announce(f"table m*2^{e} fmt={fmt} x={x_dtype}")
        y = q.moe_gemv(w, xd, to_dev(ids), values).cpu().numpy()
        assert np.all(rel_err_per_vector(y, r) <= TOL_GEMV)
        yg = q.moe_gemv_grouped(w, xd, to_dev(ids), values).cpu().numpy()
        assert np.all(rel_err_per_vector(yg, r) <= TOL_GEMV)
    # the producer takes any float32 table: bit-exact
    got = q.dequant(w, values, None, torch.float32).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), oracle.dequant(fmt, s, E * out, n, values).view(np.uint32))


def test_table_not_int8_exact_is_refused_by_the_matvec():
    w, _ = _weights(K, 2, 16, 512, 1450)
    values = np.array([1, 2, 3, 4, 5, 6, 7, 0.3], np.float32)
    x = to_dev(bf16_round(synth.normal((1, 1, 512), 1451)), torch.bfloat16)
    with pytest.raises(q.IqkError):
        q.moe_gemv(w, x, to_dev(np.array([[0]], np.int32)), values)


# ---------------------------------------------------------------------------
# IQ1_S_R4 grid values outside {-1, 0, +1}
# ---------------------------------------------------------------------------

def _int8_grid(seed):
    """2048 x 8 int8 values uniform in [-127, 127] (not a ternary grid)"""
    return np.random.default_rng(seed).integers(-127, 128, size=(2048, 8)).astype(np.int8)


def test_non_ternary_grid_float32_paths():
    E, out, n, T, k = 8, 64, 2048, 5, 3
    w, s = _weights(R4, E, out, n, 1500)
    grid = _int8_grid(1501)
    gd = to_dev(grid)
    announce("non-ternary grid: float32 producer")
    got = q.dequant(w, None, gd, torch.float32).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), oracle.dequant(R4, s, E * out, n, None, grid).view(np.uint32))
    ids = synth.topk_ids(T, k, E, 1502)
    x = bf16_round(synth.normal((T, 1, n), 1503))
    ref = oracle.moe(R4, s, E, out, n, x, ids, None, grid)
    announce("non-ternary grid: matvecs")
    y = q.moe_gemv(w, to_dev(x, torch.bfloat16), to_dev(ids), None, gd).cpu().numpy()
    assert np.all(rel_err_per_vector(y, ref) <= TOL_GEMV)
    yg = q.moe_gemv_grouped(w, to_dev(x, torch.bfloat16), to_dev(ids), None, gd).cpu().numpy()
    assert np.all(rel_err_per_vector(yg, ref) <= TOL_GEMV)


def test_non_ternary_grid_half_paths_give_nan():
    E, out, n, T, k = 8, 64, 2048, 40, 3
    w, s = _weights(R4, E, out, n, 1510)
    grid = synth.ternary_grid(1511)
    grid[977, 5] = 2  # one value off the ternary set
    gd = to_dev(grid)
    for dt in (torch.bfloat16, torch.float16):
        announce(f"non-ternary grid: producer {dt}")
        got = q.dequant(w, None, gd, dt)
        assert torch.all(torch.isnan(got)).item()
    ids = synth.topk_ids(T, k, E, 1512)
    x = to_dev(bf16_round(synth.normal((T, 1, n), 1513)), torch.bfloat16)
    announce("non-ternary grid: fused prefill")
    y = q.moe_prefill_fused(w, x, to_dev(ids), None, gd)
    assert torch.all(torch.isnan(y)).item()
    # a width the narrow producer serves (in % 64 != 0) computes every value
    w2, s2 = _weights(R4, 2, 16, 96, 1514)
    announce("non-ternary grid: narrow producer")
    got = q.dequant(w2, None, gd, torch.bfloat16).cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, oracle.dequant(R4, s2, 32, 96, None, grid, oracle.BF16))
