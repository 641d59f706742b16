"""Host-side checks of the C-ABI library (no GPU needed).

* the library loads and exports every function declared in include/iqk.h;
* iqk_row_bytes / iqk_plane_offsets agree with the row budgets of the
  "mlx-iqk" description's "Format" section;
* the host relayout is byte-exact against the oracle's relayout on random
  wires of every member, including ragged shapes;
* every validation error is returned before any HIP call (calls that would
  pass validation use T = 0 / nrows = 0, which enqueue nothing).
"""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
import synth
import dequant_iqk_moe_amd as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KS, K, R4 = 1, 2, 3


def _declared():
    src = open(os.path.join(ROOT, "include", "iqk.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(iqk_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert len(names) >= 14
    lib = ctypes.CDLL(q.library_path())
    for n in names:
        assert hasattr(lib, n), n


def test_row_bytes_and_planes():
    assert [q.row_bytes(KS, n) for n in (256, 4096)] == [72, 1122]
    assert [q.row_bytes(K, n) for n in (256, 4096)] == [76, 1216]
    assert [q.row_bytes(R4, n) for n in (32, 4096)] == [8, 770]
    assert q.row_bytes(KS, 100) == 0 and q.row_bytes(9, 256) == 0
    off, tot = q.plane_offsets(KS, 4, 256)
    assert off == [0, 256, 272, 276, 280] and tot == 288
    off, tot = q.plane_offsets(K, 2, 512)
    assert off == [0, 256, 288, 296, -1] and tot == 304
    off, tot = q.plane_offsets(R4, 4, 64)
    assert off == [0, 32, 48, -1, -1] and tot == 56


@pytest.mark.parametrize("fmt,rows,n", [(KS, 7, 512), (KS, 1, 4096), (K, 9, 768), (K, 64, 2048),
                                        (R4, 4, 32), (R4, 12, 96), (R4, 64, 4096), (KS, 0, 256)])
def test_pack_matches_oracle_bytes(fmt, rows, n):
    w = synth.random_bytes(rows * oracle.row_bytes(fmt, n), 7 + rows + fmt)
    s = q.pack_relayout(fmt, w, rows, n)
    assert np.array_equal(s, oracle.pack(fmt, w, rows, n))
    assert np.array_equal(q.unpack_relayout(fmt, s, rows, n), w)
    s2 = synth.random_bytes(w.size, 99)
    assert np.array_equal(q.unpack_relayout(fmt, s2, rows, n), oracle.unpack(fmt, s2, rows, n))


def test_pack_large_threaded_matches_oracle():
    fmt, rows, n = K, 2048, 4096          # one routed gate expert: threaded host path
    w = synth.wire(fmt, rows, n, 5)
    assert np.array_equal(q.pack_relayout(fmt, w, rows, n), oracle.pack(fmt, w, rows, n))


def _wdesc(fmt, E, out, n, nbytes=None, ptr=0x1000):
    nb = E * out * max(q.row_bytes(fmt, n), 0) if nbytes is None else nbytes
    return q._Weights(fmt, E, out, n, ptr, nb)


def _code(fn, *args):
    return fn(*args)


def test_validation_errors_before_any_launch():
    L = q._lib
    P = ctypes.c_void_p
    fake = P(0x1000)
    vals = np.arange(8, dtype=np.float32)
    vp = vals.ctypes.data_as(P)
    bad_vals = np.array([0.3] * 8, np.float32)
    s0 = P(0)
    # relayout
    buf = np.zeros(1000, np.uint8)
    bp = buf.ctypes.data_as(P)
    assert L.iqk_pack_relayout(7, bp, 72, 1, 256, bp, 72) == q._E_FORMAT
    assert L.iqk_pack_relayout(KS, bp, 72, 1, 100, bp, 72) == q._E_SHAPE
    assert L.iqk_pack_relayout(R4, bp, 98 * 3, 3, 512, P(buf.ctypes.data + 500), 98 * 3) == q._E_ROWS4
    assert L.iqk_pack_relayout(KS, bp, 71, 1, 256, P(buf.ctypes.data + 500), 72) == q._E_SIZE
    assert L.iqk_pack_relayout(KS, bp, 72, 1, 256, P(buf.ctypes.data + 10), 72) == q._E_ARG  # overlap
    assert "overlap" in L.iqk_last_error().decode()
    # matvec: width refusal ("Surface": an unsized width is refused)
    w = _wdesc(KS, 2, 8, 1024)
    assert L.iqk_moe_gemv(ctypes.byref(w), vp, None, fake, 2, 1, fake, 0, 6, fake, s0) == q._E_WIDTH
    w = _wdesc(KS, 2, 8, 2048)
    assert L.iqk_moe_gemv(ctypes.byref(w), bad_vals.ctypes.data_as(P), None, fake, 2, 1, fake, 0, 6, fake, s0) == q._E_TABLE
    assert L.iqk_moe_gemv(ctypes.byref(w), vp, None, fake, 2, 3, fake, 0, 6, fake, s0) == q._E_ARG  # x_slots
    assert L.iqk_moe_gemv(ctypes.byref(w), vp, None, fake, 1, 1, fake, 0, 6, fake, s0) == q._E_ARG  # f16 x
    w = _wdesc(KS, 2, 8, 2048, nbytes=5)
    assert L.iqk_moe_gemv(ctypes.byref(w), vp, None, fake, 2, 1, fake, 0, 6, fake, s0) == q._E_SIZE
    w = _wdesc(R4, 4, 8, 2048)
    assert L.iqk_moe_gemv(ctypes.byref(w), None, None, fake, 2, 1, fake, 0, 6, fake, s0) == q._E_ARG  # no grid
    # valid arguments with T = 0 enqueue nothing and succeed
    w = _wdesc(KS, 2, 8, 2048)
    assert L.iqk_moe_gemv(ctypes.byref(w), vp, None, fake, 2, 1, fake, 0, 6, fake, s0) == 0
    # integer-times-power-of-two tables are accepted
    halves = (np.arange(8, dtype=np.float32) - 4) * 0.5
    assert L.iqk_moe_gemv(ctypes.byref(w), halves.ctypes.data_as(P), None, fake, 2, 1, fake, 0, 6, fake, s0) == 0
    big = np.array([128, 0, 0, 0, 0, 0, 0, 1], np.float32)   # 128 * 2^0 and 1: no common exponent fits int8
    assert L.iqk_moe_gemv(ctypes.byref(w), big.ctypes.data_as(P), None, fake, 2, 1, fake, 0, 6, fake, s0) == q._E_TABLE
    # layer glue: SwiGLU needs an even gate/up row count; combine at most 8 slots
    w = _wdesc(K, 2, 9, 2048)
    assert L.iqk_moe_gemv_swiglu(ctypes.byref(w), vp, None, fake, 2, 1, fake, 0, 6, fake, s0) == q._E_SHAPE
    w = _wdesc(K, 2, 8, 2048)
    assert L.iqk_moe_gemv_swiglu(ctypes.byref(w), vp, None, fake, 2, 1, fake, 0, 6, fake, s0) == 0
    assert L.iqk_moe_gemv_combine(ctypes.byref(w), vp, None, fake, 2, 9, fake, fake, 0, 9, fake, s0) == q._E_ARG
    assert L.iqk_moe_gemv_combine(ctypes.byref(w), vp, None, fake, 2, 6, fake, None, 1, 6, fake, s0) == q._E_ARG
    assert L.iqk_moe_gemv_combine(ctypes.byref(w), vp, None, fake, 2, 6, fake, fake, 0, 6, fake, s0) == 0
    # dequant
    w = _wdesc(K, 2, 8, 512)
    assert L.iqk_dequant(ctypes.byref(w), 10, 10, vp, None, 2, fake, s0) == q._E_ARG  # rows out of range
    assert L.iqk_dequant(ctypes.byref(w), 0, 4, vp, None, 5, fake, s0) == q._E_ARG    # dtype
    assert L.iqk_dequant(ctypes.byref(w), 0, 0, vp, None, 2, fake, s0) == 0
    # route / GEMM / prefill
    assert L.iqk_route(fake, 10, 0, 0, fake, fake, fake, s0) == q._E_ARG
    assert L.iqk_route(fake, 10, 20000, 0, fake, fake, fake, s0) == q._E_ARG
    assert L.iqk_grouped_gemm(fake, 4, 64, 96, fake, 1, 0, 6, fake, fake, fake, s0) == q._E_SHAPE
    assert L.iqk_grouped_gemm(fake, 4, 60, 128, fake, 1, 0, 6, fake, fake, fake, s0) == q._E_SHAPE
    w = _wdesc(K, 4, 64, 512)
    nb = ctypes.c_size_t()
    assert L.iqk_moe_prefill_workspace(ctypes.byref(w), 8, 6, ctypes.byref(nb)) == 0
    assert nb.value == 4 * 64 * 512 * 2 + 256 + 256 + 256
    assert L.iqk_moe_prefill(ctypes.byref(w), vp, None, fake, 1, fake, 8, 6, 0, fake, nb.value - 1, fake, s0) == q._E_SIZE
    assert L.iqk_moe_prefill(ctypes.byref(w), vp, None, fake, 1, fake, 0, 6, 0, fake, nb.value, fake, s0) == 0
    # standalone glue: widths in fours, alignment
    assert L.iqk_swiglu(fake, 4, 6, fake, s0) == q._E_SHAPE
    assert L.iqk_swiglu(P(0x1008), 4, 8, fake, s0) == q._E_ARG
    assert L.iqk_swiglu(fake, 0, 8, None, s0) == 0
    assert L.iqk_combine(fake, fake, 2, 6, 10, fake, s0) == q._E_SHAPE
    assert L.iqk_combine(fake, fake, 2, 0, 8, fake, s0) == q._E_ARG
    assert L.iqk_combine(fake, fake, 0, 6, 8, fake, s0) == 0
    # fused prefill and grouped matvec: routing arrays plus an int64 [E + 1] work plan
    assert L.iqk_moe_prefill_fused_workspace(ctypes.byref(w), 8, 6, ctypes.byref(nb)) == 0
    assert nb.value == 256 + 256 + 256 + 256
    w = _wdesc(K, 4, 64, 2048)
    assert L.iqk_moe_gemv_grouped_workspace(ctypes.byref(w), 100, 6, ctypes.byref(nb)) == 0
    assert nb.value == 256 + 256 + 2560 + 256
    assert L.iqk_moe_gemv_grouped(ctypes.byref(w), vp, None, fake, 2, 1, fake, 100, 6, 0, fake, nb.value - 1, fake,
                                  s0) == q._E_SIZE
    assert L.iqk_moe_gemv_grouped(ctypes.byref(w), vp, None, fake, 2, 1, fake, 100, 6, 2, fake, nb.value, fake,
                                  s0) == q._E_ARG  # sorted flag
    assert L.iqk_moe_gemv_grouped(ctypes.byref(w), bad_vals.ctypes.data_as(P), None, fake, 2, 1, fake, 100, 6, 0,
                                  fake, nb.value, fake, s0) == q._E_TABLE
    assert L.iqk_moe_gemv_grouped(ctypes.byref(w), vp, None, fake, 2, 1, fake, 0, 6, 0, fake, nb.value, fake,
                                  s0) == 0
    w = _wdesc(K, 4, 64, 1024)
    assert L.iqk_moe_gemv_grouped(ctypes.byref(w), vp, None, fake, 2, 1, fake, 1, 6, 0, fake, 1 << 20, fake,
                                  s0) == q._E_WIDTH
    # plain streaming write: sizes in 16 bytes, 1..16 runs per wave
    assert L.iqk_stream_write(fake, 100, 0, 1, s0) == q._E_ARG
    assert L.iqk_stream_write(fake, 4096, 0, 0, s0) == q._E_ARG
    assert L.iqk_stream_write(fake, 4096, 0, 17, s0) == q._E_ARG


def test_python_errors_map_to_exception_types():
    with pytest.raises(q.IqkValueError):
        q.pack_relayout(R4, np.zeros(3 * 98, np.uint8), 3, 512)
    with pytest.raises(q.IqkValueError):
        q.plane_offsets(KS, 4, 100)


def test_package_refuses_to_import_without_the_library(tmp_path):
    """no CPU fallback: a copy of the package without libiqk.so fails to import"""
    import shutil
    import subprocess
    import sys
    src = os.path.dirname(q.__file__)
    dst = tmp_path / "dequant_iqk_moe_amd"
    shutil.copytree(src, dst, ignore=shutil.ignore_patterns("*.so", "_build", "__pycache__"))
    r = subprocess.run([sys.executable, "-c", "import dequant_iqk_moe_amd"], cwd=tmp_path, capture_output=True,
                       text=True, env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode != 0 and "ImportError" in r.stderr and "not built" in r.stderr
