"""IQ_K routed-expert kernels for MI355X -- thin Python binding over ``libiqk.so``.

Every call here is argument marshalling for the C ABI declared in
``include/iqk.h`` (same names without the ``iqk_`` prefix).  All arithmetic
runs in the library's HIP kernels (or its host relayout); PyTorch supplies
device memory and the current stream only.  If ``libiqk.so`` has not been
built, importing this package raises ``ImportError`` -- there is no CPU
fallback.

Operations follow the "mlx-iqk" package description: the relayout of
"Format" (``pack_relayout`` / ``unpack_relayout``), the float32
reconstruction of "Format" (``dequant``), and the switch-linear call of
"Surface" (``moe_gemv`` for few token-expert pairs, ``moe_prefill`` =
``route`` + ``dequant`` + ``grouped_gemm`` for many).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

__all__ = [
    "IQ2_KS", "IQ2_K", "IQ1_S_R4", "IqkError", "IqkValueError", "Weights",
    "row_bytes", "plane_offsets", "pack_relayout", "unpack_relayout", "dequant", "moe_gemv",
    "route", "grouped_gemm", "prefill_workspace_bytes", "moe_prefill", "floor_gemv",
    "floor_dequant", "stream_read", "stream_write", "library_path",
]

IQ2_KS, IQ2_K, IQ1_S_R4 = 1, 2, 3
FORMAT_NAMES = {"iq2_ks": IQ2_KS, "iq2_k": IQ2_K, "iq1_s_r4": IQ1_S_R4}
_F32, _F16, _BF16 = 0, 1, 2
_DT = {torch.float32: _F32, torch.float16: _F16, torch.bfloat16: _BF16}

_E_ARG, _E_FORMAT, _E_SHAPE, _E_WIDTH, _E_ROWS4, _E_SIZE, _E_TABLE, _E_HIP = -1, -2, -3, -4, -5, -6, -7, -8
_VALUE_ERRORS = {_E_ARG, _E_FORMAT, _E_SHAPE, _E_ROWS4, _E_SIZE}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libiqk.so")


class IqkError(RuntimeError):
    """Unsupported request (no instance for a width, table not int8-exact) or a HIP error."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"[iqk {code}] {msg}")
        self.code = code


class IqkValueError(ValueError):
    """Bad arguments: format, shape, sizes, row groups."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"[iqk {code}] {msg}")
        self.code = code


class _Weights(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("experts", ctypes.c_int64), ("out", ctypes.c_int64),
                ("in_", ctypes.c_int64), ("streams", ctypes.c_void_p), ("streams_bytes", ctypes.c_size_t)]


def library_path() -> str:
    return _LIB_PATH


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python dequant_iqk_moe_amd/build.py`")
    L = ctypes.CDLL(_LIB_PATH)
    p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    W = ctypes.POINTER(_Weights)
    sig = {
        "iqk_row_bytes": (sz, [i32, i64]),
        "iqk_plane_offsets": (i32, [i32, i64, i64, p, p]),
        "iqk_pack_relayout": (i32, [i32, p, sz, i64, i64, p, sz]),
        "iqk_unpack_relayout": (i32, [i32, p, sz, i64, i64, p, sz]),
        "iqk_dequant": (i32, [W, i64, i64, p, p, i32, p, p]),
        "iqk_moe_gemv": (i32, [W, p, p, p, i32, i32, p, i64, i32, p, p]),
        "iqk_moe_gemv_swiglu": (i32, [W, p, p, p, i32, i32, p, i64, i32, p, p]),
        "iqk_moe_gemv_combine": (i32, [W, p, p, p, i32, i32, p, p, i64, i32, p, p]),
        "iqk_moe_gemv_grouped_workspace": (i32, [W, i64, i32, p]),
        "iqk_moe_gemv_grouped": (i32, [W, p, p, p, i32, i32, p, i64, i32, i32, p, sz, p, p]),
        "iqk_moe_auto_workspace": (i32, [W, i64, i32, p]),
        "iqk_moe_auto": (i32, [W, p, p, p, i32, i32, p, i64, i32, p, sz, p, p, p]),
        "iqk_moe_auto_noalloc": (i32, [W, p, p, p, i32, i32, p, i64, i32, p, p, p]),
        "iqk_swiglu": (i32, [p, i64, i64, p, p]),
        "iqk_combine": (i32, [p, p, i64, i32, i64, p, p]),
        "iqk_route": (i32, [p, i64, i64, i32, p, p, p, p]),
        "iqk_grouped_gemm": (i32, [p, i64, i64, i64, p, i32, i64, i32, p, p, p, p]),
        "iqk_moe_prefill_workspace": (i32, [W, i64, i32, p]),
        "iqk_moe_prefill": (i32, [W, p, p, p, i32, p, i64, i32, i32, p, sz, p, p]),
        "iqk_moe_prefill_fused_workspace": (i32, [W, i64, i32, p]),
        "iqk_moe_prefill_fused": (i32, [W, p, p, p, i32, p, i64, i32, i32, p, sz, p, p]),
        "iqk_floor_gemv": (i32, [W, p, p, p, i32, i32, p, i64, i32, p, p]),
        "iqk_floor_dequant": (i32, [W, i64, i64, i32, p, p]),
        "iqk_stream_read": (i32, [p, sz, p, sz, p]),
        "iqk_stream_write": (i32, [p, sz, ctypes.c_uint32, i32, p]),
        "iqk_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


_lib = _load()


def _check(rc: int):
    if rc == 0:
        return
    msg = _lib.iqk_last_error().decode()
    if rc in _VALUE_ERRORS:
        raise IqkValueError(rc, msg)
    raise IqkError(rc, msg)


def _fmt(fmt) -> int:
    if isinstance(fmt, str):
        return FORMAT_NAMES[fmt.lower()]
    return int(fmt)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


GRID_NUMEL = 2048 * 8  # the IQ1_S_R4 grid: 2048 entries of 8 int8 values


def _dev(t: torch.Tensor | None, what: str, dtype=None, numel: int | None = None):
    """Device pointer of a contiguous tensor, after checking its dtype and,
    when `numel` is given, its element count (the kernels read or write
    exactly that many elements; a shorter buffer would be overrun)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise IqkValueError(_E_ARG, f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise IqkValueError(_E_ARG, f"{what} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise IqkValueError(_E_ARG, f"{what} must be {dtype}, got {t.dtype}")
    if numel is not None and t.numel() != numel:
        raise IqkValueError(_E_SIZE, f"{what} has {t.numel()} elements, expected {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _grid(grid: torch.Tensor | None):
    return _dev(grid, "grid", torch.int8, GRID_NUMEL)


def _ids(ids: torch.Tensor):
    if ids.dim() != 2:
        raise IqkValueError(_E_ARG, "ids must be [T, k]")
    return _dev(ids, "ids", torch.int32)


def _host_values(values):
    if values is None:
        return None, None
    v = np.ascontiguousarray(np.asarray(values, np.float32).ravel())
    if v.size != 8:
        raise IqkValueError(_E_ARG, "the value table has 8 entries")
    return v, v.ctypes.data_as(ctypes.c_void_p)


def row_bytes(fmt, n: int) -> int:
    return int(_lib.iqk_row_bytes(_fmt(fmt), n))


def plane_offsets(fmt, rows: int, n: int):
    off = (ctypes.c_int64 * 5)()
    tot = ctypes.c_int64()
    _check(_lib.iqk_plane_offsets(_fmt(fmt), rows, n, off, ctypes.byref(tot)))
    return list(off), tot.value


def pack_relayout(fmt, wire: np.ndarray, rows: int, n: int) -> np.ndarray:
    """Host relayout wire -> canonical streams (byte-exact permutation)."""
    w = np.ascontiguousarray(wire, np.uint8).ravel()
    out = np.empty(w.size, np.uint8)
    _check(_lib.iqk_pack_relayout(_fmt(fmt), w.ctypes.data_as(ctypes.c_void_p), w.size, rows, n,
                                  out.ctypes.data_as(ctypes.c_void_p), out.size))
    return out


def unpack_relayout(fmt, streams: np.ndarray, rows: int, n: int) -> np.ndarray:
    s = np.ascontiguousarray(streams, np.uint8).ravel()
    out = np.empty(s.size, np.uint8)
    _check(_lib.iqk_unpack_relayout(_fmt(fmt), s.ctypes.data_as(ctypes.c_void_p), s.size, rows, n,
                                    out.ctypes.data_as(ctypes.c_void_p), out.size))
    return out


@dataclass
class Weights:
    """Expert-stacked stream tensor: `experts` x [out, in_features] in one
    device uint8 tensor laid out as the canonical streams."""

    fmt: int
    experts: int
    out: int
    in_features: int
    streams: torch.Tensor

    @staticmethod
    def from_wire(fmt, experts: int, out: int, in_features: int, wire: np.ndarray, device="cuda") -> "Weights":
        s = pack_relayout(fmt, wire, experts * out, in_features)
        return Weights(_fmt(fmt), experts, out, in_features, torch.from_numpy(s).to(device))

    def _c(self) -> _Weights:
        if not self.streams.is_cuda or self.streams.dtype != torch.uint8 or not self.streams.is_contiguous():
            raise IqkValueError(_E_ARG, "streams must be a contiguous device uint8 tensor")
        return _Weights(_fmt(self.fmt), self.experts, self.out, self.in_features,
                        self.streams.data_ptr(), self.streams.numel())


def dequant(w: Weights, values=None, grid: torch.Tensor | None = None, out_dtype=torch.float32,
            row0: int = 0, nrows: int | None = None, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    nrows = w.experts * w.out - row0 if nrows is None else nrows
    if out is None:
        out = torch.empty((nrows, w.in_features), dtype=out_dtype, device=w.streams.device)
    _v, vp = _host_values(values)
    cw = w._c()
    if out.dtype not in _DT:
        raise IqkValueError(_E_ARG, "out must be float32, float16 or bfloat16")
    _check(_lib.iqk_dequant(ctypes.byref(cw), row0, nrows, vp, _grid(grid),
                            _DT[out.dtype], _dev(out, "out", numel=nrows * w.in_features), _stream(stream)))
    return out


def _x_args(x: torch.Tensor, T: int, x_slots: int, n: int):
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise IqkValueError(_E_ARG, "x must be float32 or bfloat16")
    if x.numel() != T * x_slots * n:
        raise IqkValueError(_E_SIZE, f"x has {x.numel()} elements, expected T*x_slots*in = {T * x_slots * n}")
    return _dev(x, "x"), _DT[x.dtype]


def moe_gemv(w: Weights, x: torch.Tensor, ids: torch.Tensor, values=None, grid: torch.Tensor | None = None,
             x_slots: int = 1, y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Fused decode matvec: y[T, k, out] (float32)."""
    T, k = ids.shape
    xp, xdt = _x_args(x, T, x_slots, w.in_features)
    if y is None:
        y = torch.empty((T, k, w.out), dtype=torch.float32, device=w.streams.device)
    _v, vp = _host_values(values)
    cw = w._c()
    _check(_lib.iqk_moe_gemv(ctypes.byref(cw), vp, _grid(grid), xp, xdt, x_slots,
                             _ids(ids), T, k, _dev(y, "y", torch.float32, T * k * w.out), _stream(stream)))
    return y


def moe_gemv_swiglu(w: Weights, x: torch.Tensor, ids: torch.Tensor, values=None, grid: torch.Tensor | None = None,
                    x_slots: int = 1, h: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Gate/up matvec with the SwiGLU epilogue: h[T, k, out // 2] (bf16),
    h = silu(gate) * up with gate rows [0, I) and up rows [I, 2I)."""
    T, k = ids.shape
    xp, xdt = _x_args(x, T, x_slots, w.in_features)
    if h is None:
        h = torch.empty((T, k, w.out // 2), dtype=torch.bfloat16, device=w.streams.device)
    _v, vp = _host_values(values)
    cw = w._c()
    _check(_lib.iqk_moe_gemv_swiglu(ctypes.byref(cw), vp, _grid(grid), xp, xdt, x_slots,
                                    _ids(ids), T, k, _dev(h, "h", torch.bfloat16, T * k * (w.out // 2)),
                                    _stream(stream)))
    return h


def moe_gemv_combine(w: Weights, x: torch.Tensor, ids: torch.Tensor, route_w: torch.Tensor, values=None,
                     grid: torch.Tensor | None = None, x_slots: int | None = None, y: torch.Tensor | None = None,
                     stream=None) -> torch.Tensor:
    """Down matvec with the router-weighted combine: y[T, out] (float32),
    y[t] = sum_j route_w[t, j] * W_{ids[t, j]} x[t, j].  x_slots defaults to k."""
    T, k = ids.shape
    x_slots = k if x_slots is None else x_slots
    xp, xdt = _x_args(x, T, x_slots, w.in_features)
    if y is None:
        y = torch.empty((T, w.out), dtype=torch.float32, device=w.streams.device)
    _v, vp = _host_values(values)
    cw = w._c()
    _check(_lib.iqk_moe_gemv_combine(ctypes.byref(cw), vp, _grid(grid), xp, xdt, x_slots,
                                     _ids(ids), _dev(route_w, "route_w", torch.float32, T * k), T, k,
                                     _dev(y, "y", torch.float32, T * w.out), _stream(stream)))
    return y


def gemv_grouped_workspace_bytes(w: Weights, T: int, k: int) -> int:
    b = ctypes.c_size_t()
    cw = _Weights(_fmt(w.fmt), w.experts, w.out, w.in_features, None, 0)
    _check(_lib.iqk_moe_gemv_grouped_workspace(ctypes.byref(cw), T, k, ctypes.byref(b)))
    return b.value


def moe_gemv_grouped(w: Weights, x: torch.Tensor, ids: torch.Tensor, values=None, grid: torch.Tensor | None = None,
                     x_slots: int = 1, sorted: bool = False, workspace: torch.Tensor | None = None,
                     y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Grouped decode matvec: route, then one decode pass per selected expert
    shared by all of its pairs.  y[T, k, out] (float32); pairs with an
    invalid id get NaN rows."""
    T, k = ids.shape
    xp, xdt = _x_args(x, T, x_slots, w.in_features)
    if workspace is None:
        workspace = torch.empty(gemv_grouped_workspace_bytes(w, T, k), dtype=torch.uint8, device=w.streams.device)
    if y is None:
        y = torch.zeros((T, k, w.out), dtype=torch.float32, device=w.streams.device)
    _v, vp = _host_values(values)
    cw = w._c()
    _check(_lib.iqk_moe_gemv_grouped(ctypes.byref(cw), vp, _grid(grid), xp, xdt, x_slots,
                                     _ids(ids), T, k, int(bool(sorted)),
                                     _dev(workspace, "workspace", torch.uint8), workspace.numel(),
                                     _dev(y, "y", torch.float32, T * k * w.out), _stream(stream)))
    return y


def swiglu(y_gu: torch.Tensor, h: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """h = silu(gate) * up (bf16) from a gate/up projection's output
    y_gu [..., 2I] (float32; gate columns first)."""
    if y_gu.dtype != torch.float32 or y_gu.shape[-1] % 2:
        raise IqkValueError(_E_ARG, "y_gu must be float32 [..., 2I]")
    I = y_gu.shape[-1] // 2
    P = y_gu.numel() // (2 * I)
    if h is None:
        h = torch.empty((*y_gu.shape[:-1], I), dtype=torch.bfloat16, device=y_gu.device)
    _check(_lib.iqk_swiglu(_dev(y_gu, "y_gu", torch.float32), P, I, _dev(h, "h", torch.bfloat16, P * I),
                           _stream(stream)))
    return h


def combine(y: torch.Tensor, route_w: torch.Tensor, yc: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """yc[t] = sum_j route_w[t, j] * y[t, j] (float32, slot order) from y [T, k, out]."""
    T, k, out = y.shape
    if yc is None:
        yc = torch.empty((T, out), dtype=torch.float32, device=y.device)
    _check(_lib.iqk_combine(_dev(y, "y", torch.float32), _dev(route_w, "route_w", torch.float32, T * k), T, k, out,
                            _dev(yc, "yc", torch.float32, T * out), _stream(stream)))
    return yc


AUTO_PATHS = ("gemv", "grouped_gemv", "fused_prefill")


def moe_auto(w: Weights, x: torch.Tensor, ids: torch.Tensor, values=None, grid: torch.Tensor | None = None,
             x_slots: int = 1, workspace: torch.Tensor | None = None, y: torch.Tensor | None = None,
             stream=None) -> tuple[torch.Tensor, str]:
    """The routed projection with the path picked by pairs per expert
    (per-pair matvec, grouped matvec or fused prefill); returns (y, path)."""
    T, k = ids.shape
    xp, xdt = _x_args(x, T, x_slots, w.in_features)
    if workspace is None:
        b = ctypes.c_size_t()
        cw0 = _Weights(_fmt(w.fmt), w.experts, w.out, w.in_features, None, 0)
        _check(_lib.iqk_moe_auto_workspace(ctypes.byref(cw0), T, k, ctypes.byref(b)))
        workspace = torch.empty(b.value, dtype=torch.uint8, device=w.streams.device)
    if y is None:
        y = torch.zeros((T, k, w.out), dtype=torch.float32, device=w.streams.device)
    _v, vp = _host_values(values)
    cw = w._c()
    path = ctypes.c_int(-1)
    _check(_lib.iqk_moe_auto(ctypes.byref(cw), vp, _grid(grid), xp, xdt, x_slots,
                             _ids(ids), T, k, _dev(workspace, "workspace", torch.uint8),
                             workspace.numel(), _dev(y, "y", torch.float32, T * k * w.out), ctypes.byref(path),
                             _stream(stream)))
    return y, AUTO_PATHS[path.value]


def moe_auto_noalloc(w: Weights, x: torch.Tensor, ids: torch.Tensor, y: torch.Tensor, values=None,
                     grid: torch.Tensor | None = None, x_slots: int = 1, stream=None) -> str:
    """moe_auto without a workspace and without any allocation: the
    library's fixed device scratch holds the routing arrays (calls that
    overlap on one GPU race).  y [T, k, out] float32 is the caller's;
    returns the path taken."""
    T, k = ids.shape
    xp, xdt = _x_args(x, T, x_slots, w.in_features)
    _v, vp = _host_values(values)
    cw = w._c()
    path = ctypes.c_int(-1)
    _check(_lib.iqk_moe_auto_noalloc(ctypes.byref(cw), vp, _grid(grid), xp, xdt, x_slots, _ids(ids), T, k,
                                     _dev(y, "y", torch.float32, T * k * w.out), ctypes.byref(path),
                                     _stream(stream)))
    return AUTO_PATHS[path.value]


def floor_gemv(w: Weights, x: torch.Tensor, ids: torch.Tensor, values=None, grid: torch.Tensor | None = None,
               x_slots: int = 1, sink: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Deleted-decode floor of moe_gemv (same loads; integer accumulator out)."""
    T, k = ids.shape
    xp, xdt = _x_args(x, T, x_slots, w.in_features)
    if sink is None:
        sink = torch.empty((T, k, w.out), dtype=torch.int32, device=w.streams.device)
    _v, vp = _host_values(values)
    cw = w._c()
    _check(_lib.iqk_floor_gemv(ctypes.byref(cw), vp, _grid(grid), xp, xdt, x_slots,
                               _ids(ids), T, k, _dev(sink, "sink", torch.int32, T * k * w.out),
                               _stream(stream)))
    return sink


def floor_dequant(w: Weights, out_dtype=torch.bfloat16, row0: int = 0, nrows: int | None = None,
                  out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    nrows = w.experts * w.out - row0 if nrows is None else nrows
    if out is None:
        out = torch.empty((nrows, w.in_features), dtype=out_dtype, device=w.streams.device)
    cw = w._c()
    if out.dtype not in _DT:
        raise IqkValueError(_E_ARG, "out must be float32, float16 or bfloat16")
    _check(_lib.iqk_floor_dequant(ctypes.byref(cw), row0, nrows, _DT[out.dtype],
                                  _dev(out, "out", numel=nrows * w.in_features), _stream(stream)))
    return out


def stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> torch.Tensor:
    nbytes = buf.numel() * buf.element_size()
    _check(_lib.iqk_stream_read(_dev(buf, "buf"), nbytes, _dev(sink, "sink", torch.int32), sink.numel(),
                                _stream(stream)))
    return sink


def stream_write(buf: torch.Tensor, value: int = 0, runs: int = 1, stream=None) -> torch.Tensor:
    """Plain streaming write of `value` into every 32-bit word of buf (the
    write ceiling of the dequantization producer); each wave writes `runs`
    consecutive 1 KiB runs (1: the fastest shape, 8: the bf16 producer's)."""
    nbytes = buf.numel() * buf.element_size()
    _check(_lib.iqk_stream_write(_dev(buf, "buf"), nbytes, int(value) & 0xFFFFFFFF, int(runs), _stream(stream)))
    return buf


def route(ids: torch.Tensor, E: int, sorted: bool = False, stream=None):
    """Stable expert sort of the pairs: (counts[E], offsets[E+1], perm[P]) int32 device tensors."""
    P = ids.numel()
    dev = ids.device
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(P, 1), dtype=torch.int32, device=dev)
    _check(_lib.iqk_route(_dev(ids, "ids", torch.int32), P, E, int(bool(sorted)), _dev(counts, "counts"),
                          _dev(offsets, "offsets"), _dev(perm, "perm"), _stream(stream)))
    return counts, offsets, perm[:P]


def grouped_gemm(W: torch.Tensor, x: torch.Tensor, T: int, k: int, offsets: torch.Tensor, perm: torch.Tensor,
                 x_slots: int = 1, y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """MFMA grouped GEMM over dense bf16 experts W [E, out, in] for routed pairs."""
    E, out, n = W.shape
    if x.dtype != torch.bfloat16 or x.numel() != T * x_slots * n:
        raise IqkValueError(_E_SIZE, "x must be bf16 [T, x_slots, in]")
    if y is None:
        y = torch.zeros((T, k, out), dtype=torch.float32, device=W.device)
    if perm.numel() < T * k:
        raise IqkValueError(_E_SIZE, f"perm has {perm.numel()} elements, expected at least T*k = {T * k}")
    _check(_lib.iqk_grouped_gemm(_dev(W, "W", torch.bfloat16), E, out, n, _dev(x, "x"), x_slots, T, k,
                                 _dev(offsets, "offsets", torch.int32, E + 1), _dev(perm, "perm", torch.int32),
                                 _dev(y, "y", torch.float32, T * k * out), _stream(stream)))
    return y


def prefill_workspace_bytes(w: Weights, T: int, k: int) -> int:
    b = ctypes.c_size_t()
    cw = _Weights(_fmt(w.fmt), w.experts, w.out, w.in_features, None, 0)
    _check(_lib.iqk_moe_prefill_workspace(ctypes.byref(cw), T, k, ctypes.byref(b)))
    return b.value


def moe_prefill(w: Weights, x: torch.Tensor, ids: torch.Tensor, values=None, grid: torch.Tensor | None = None,
                x_slots: int = 1, sorted: bool = False, workspace: torch.Tensor | None = None,
                y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Prefill: route + one-pass dequant of all experts to bf16 + MFMA grouped GEMM."""
    T, k = ids.shape
    if x.dtype != torch.bfloat16 or x.numel() != T * x_slots * w.in_features:
        raise IqkValueError(_E_SIZE, "x must be bf16 [T, x_slots, in]")
    if workspace is None:
        workspace = torch.empty(prefill_workspace_bytes(w, T, k), dtype=torch.uint8, device=w.streams.device)
    if y is None:
        y = torch.zeros((T, k, w.out), dtype=torch.float32, device=w.streams.device)
    _v, vp = _host_values(values)
    cw = w._c()
    _check(_lib.iqk_moe_prefill(ctypes.byref(cw), vp, _grid(grid), _dev(x, "x"), x_slots,
                                _ids(ids), T, k, int(bool(sorted)),
                                _dev(workspace, "workspace", torch.uint8), workspace.numel(),
                                _dev(y, "y", torch.float32, T * k * w.out), _stream(stream)))
    return y


def prefill_fused_workspace_bytes(w: Weights, T: int, k: int) -> int:
    b = ctypes.c_size_t()
    cw = _Weights(_fmt(w.fmt), w.experts, w.out, w.in_features, None, 0)
    _check(_lib.iqk_moe_prefill_fused_workspace(ctypes.byref(cw), T, k, ctypes.byref(b)))
    return b.value


def moe_prefill_fused(w: Weights, x: torch.Tensor, ids: torch.Tensor, values=None, grid: torch.Tensor | None = None,
                      x_slots: int = 1, sorted: bool = False, workspace: torch.Tensor | None = None,
                      y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Prefill with the dequantization fused into the MFMA grouped GEMM
    (route + one kernel; no dense weight copy)."""
    T, k = ids.shape
    if x.dtype != torch.bfloat16 or x.numel() != T * x_slots * w.in_features:
        raise IqkValueError(_E_SIZE, "x must be bf16 [T, x_slots, in]")
    if workspace is None:
        workspace = torch.empty(prefill_fused_workspace_bytes(w, T, k), dtype=torch.uint8, device=w.streams.device)
    if y is None:
        y = torch.zeros((T, k, w.out), dtype=torch.float32, device=w.streams.device)
    _v, vp = _host_values(values)
    cw = w._c()
    _check(_lib.iqk_moe_prefill_fused(ctypes.byref(cw), vp, _grid(grid), _dev(x, "x"), x_slots,
                                      _ids(ids), T, k, int(bool(sorted)),
                                      _dev(workspace, "workspace", torch.uint8), workspace.numel(),
                                      _dev(y, "y", torch.float32, T * k * w.out), _stream(stream)))
    return y
