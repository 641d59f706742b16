"""CPU oracle for the IQ_K routed-expert path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product package
``dequant_iqk_moe_amd`` never imports it and shares no code with it.

The arithmetic lives in ``iqk_oracle.c`` (plain scalar C, float32
reconstruction chain in the order the "mlx-iqk" package description's
"Format" section gives, double accumulation for products).  This module is
argument marshalling only.

MoE-layer glue on either side of the projections (``swiglu``, ``combine``)
is not on the pages: it is the standard SwiGLU expert MLP and the
router-weighted sum of the routed experts, written here as their plain
float64 definitions in numpy.

Parity pins: every function here is checked in ``tests/test_oracle_*.py``
against hand-computed blocks, exact closed forms, library routines (numpy /
torch casts, numpy float64 matmul, numpy stable argsort) and bijection
properties.  Equality with real ik_llama wire bytes, the real ``iq2nl_values``
table and the real IQ1_S grid is *parity unpinned* (none of them is available).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "iqk_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

IQ2_KS, IQ2_K, IQ1_S_R4 = 1, 2, 3
F32, F16, BF16 = 0, 1, 2

FIELD_DTYPE = np.dtype([("d", "<u2"), ("a", "<i2"), ("b", "<i2"), ("c", "<i2")])

_CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (strict IEEE float32: no FMA contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        i64, i32, p = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
        L.orc_f16_to_f32.restype = ctypes.c_float
        L.orc_f16_to_f32.argtypes = [ctypes.c_uint16]
        L.orc_f32_to_f16.restype = ctypes.c_uint16
        L.orc_f32_to_f16.argtypes = [ctypes.c_float]
        L.orc_f32_to_bf16.restype = ctypes.c_uint16
        L.orc_f32_to_bf16.argtypes = [ctypes.c_float]
        for name in ("orc_f16_to_f32_n", "orc_f32_to_f16_n", "orc_f32_to_bf16_n"):
            fn = getattr(L, name)
            fn.restype = None
            fn.argtypes = [p, p, i64]
        L.orc_row_bytes.restype = i64
        L.orc_row_bytes.argtypes = [i32, i64]
        L.orc_tensor_bytes.restype = i64
        L.orc_tensor_bytes.argtypes = [i32, i64, i64]
        for name in ("orc_decode_streams", "orc_decode_wire"):
            fn = getattr(L, name)
            fn.restype = i32
            fn.argtypes = [i32, p, i64, i64, i64, i64, p]
        for name in ("orc_encode_streams", "orc_encode_wire"):
            fn = getattr(L, name)
            fn.restype = i32
            fn.argtypes = [i32, p, i64, i64, p]
        for name in ("orc_pack", "orc_unpack"):
            fn = getattr(L, name)
            fn.restype = i32
            fn.argtypes = [i32, p, i64, i64, p]
        L.orc_dequant.restype = i32
        L.orc_dequant.argtypes = [i32, p, i64, i64, i64, i64, p, p, i32, p]
        L.orc_moe.restype = i32
        L.orc_moe.argtypes = [i32, p, i64, i64, i64, p, p, p, i64, p, i64, i64, i32, p]
        L.orc_route.restype = i64
        L.orc_route.argtypes = [p, i64, i64, p, p, p]
        _lib = L
    return _lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def f16_to_f32(h: int) -> float:
    return lib().orc_f16_to_f32(int(h))


def f32_to_f16_bits(f: float) -> int:
    return lib().orc_f32_to_f16(float(f))


def f32_to_bf16_bits(f: float) -> int:
    return lib().orc_f32_to_bf16(float(f))


def f16_to_f32_array(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, np.uint16).ravel()
    out = np.empty(h.size, np.float32)
    lib().orc_f16_to_f32_n(_ptr(h), _ptr(out), h.size)
    return out


def f32_to_f16_array(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32).ravel()
    out = np.empty(x.size, np.uint16)
    lib().orc_f32_to_f16_n(_ptr(x), _ptr(out), x.size)
    return out


def f32_to_bf16_array(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, np.float32).ravel()
    out = np.empty(x.size, np.uint16)
    lib().orc_f32_to_bf16_n(_ptr(x), _ptr(out), x.size)
    return out


def row_bytes(fmt: int, n: int) -> int:
    return int(lib().orc_row_bytes(fmt, n))


def tensor_bytes(fmt: int, rows: int, n: int) -> int:
    return int(lib().orc_tensor_bytes(fmt, rows, n))


def decode_streams(fmt: int, streams: np.ndarray, rows: int, n: int, r0: int = 0, nr: int | None = None) -> np.ndarray:
    nr = rows - r0 if nr is None else nr
    f = np.zeros(nr * n, FIELD_DTYPE)
    s = np.ascontiguousarray(streams, np.uint8)
    _check(lib().orc_decode_streams(fmt, _ptr(s), rows, n, r0, nr, _ptr(f)), "decode_streams")
    return f.reshape(nr, n)


def decode_wire(fmt: int, wire: np.ndarray, rows: int, n: int, r0: int = 0, nr: int | None = None) -> np.ndarray:
    nr = rows - r0 if nr is None else nr
    f = np.zeros(nr * n, FIELD_DTYPE)
    w = np.ascontiguousarray(wire, np.uint8)
    _check(lib().orc_decode_wire(fmt, _ptr(w), rows, n, r0, nr, _ptr(f)), "decode_wire")
    return f.reshape(nr, n)


def encode_streams(fmt: int, fields: np.ndarray, rows: int, n: int) -> np.ndarray:
    f = np.ascontiguousarray(fields.reshape(-1), FIELD_DTYPE)
    out = np.zeros(rows * row_bytes(fmt, n), np.uint8)
    _check(lib().orc_encode_streams(fmt, _ptr(f), rows, n, _ptr(out)), "encode_streams")
    return out


def encode_wire(fmt: int, fields: np.ndarray, rows: int, n: int) -> np.ndarray:
    f = np.ascontiguousarray(fields.reshape(-1), FIELD_DTYPE)
    out = np.zeros(rows * row_bytes(fmt, n), np.uint8)
    _check(lib().orc_encode_wire(fmt, _ptr(f), rows, n, _ptr(out)), "encode_wire")
    return out


def pack(fmt: int, wire: np.ndarray, rows: int, n: int) -> np.ndarray:
    w = np.ascontiguousarray(wire, np.uint8)
    if w.size != rows * row_bytes(fmt, n):
        raise ValueError("wire size does not match the row budget")
    out = np.zeros(w.size, np.uint8)
    _check(lib().orc_pack(fmt, _ptr(w), rows, n, _ptr(out)), "pack")
    return out


def unpack(fmt: int, streams: np.ndarray, rows: int, n: int) -> np.ndarray:
    s = np.ascontiguousarray(streams, np.uint8)
    if s.size != rows * row_bytes(fmt, n):
        raise ValueError("stream size does not match the row budget")
    out = np.zeros(s.size, np.uint8)
    _check(lib().orc_unpack(fmt, _ptr(s), rows, n, _ptr(out)), "unpack")
    return out


def _values(values):
    if values is None:
        return None
    v = np.ascontiguousarray(values, np.float32)
    assert v.size == 8
    return v


def _grid(grid):
    if grid is None:
        return None
    g = np.ascontiguousarray(grid, np.int8)
    assert g.size == 2048 * 8
    return g


def dequant(fmt: int, streams: np.ndarray, rows: int, n: int, values=None, grid=None,
            dtype: int = F32, r0: int = 0, nr: int | None = None) -> np.ndarray:
    """float32 chain per weight; f16/bf16 results are returned as uint16 bit patterns."""
    nr = rows - r0 if nr is None else nr
    s = np.ascontiguousarray(streams, np.uint8)
    v, g = _values(values), _grid(grid)
    out = np.zeros(nr * n, np.float32 if dtype == F32 else np.uint16)
    _check(lib().orc_dequant(fmt, _ptr(s), rows, n, r0, nr, _ptr(v), _ptr(g), dtype, _ptr(out)), "dequant")
    return out.reshape(nr, n)


def weight_rows(fmt: int, fields: np.ndarray, values=None, grid=None) -> np.ndarray:
    """Reconstruct float32 weights from decoded fields (rows x n) by streams re-encoding."""
    rows, n = fields.shape
    s = encode_streams(fmt, fields, rows, n)
    return dequant(fmt, s, rows, n, values, grid, F32)


def moe(fmt: int, streams: np.ndarray, E: int, out: int, n: int, x: np.ndarray, ids: np.ndarray,
        values=None, grid=None, x_slots: int = 1, w_bf16: bool = False) -> np.ndarray:
    """y[T, k, out] (float64) of the routed-expert product, x given as [T, x_slots, n]."""
    ids = np.ascontiguousarray(ids, np.int32)
    T, k = ids.shape
    xd = np.ascontiguousarray(np.asarray(x, np.float64).reshape(T, x_slots, n))
    s = np.ascontiguousarray(streams, np.uint8)
    y = np.zeros((T, k, out), np.float64)
    _check(lib().orc_moe(fmt, _ptr(s), E, out, n, _ptr(_values(values)), _ptr(_grid(grid)),
                         _ptr(xd), x_slots, _ptr(ids), T, k, int(bool(w_bf16)), _ptr(y)), "moe")
    return y


def route(ids: np.ndarray, E: int):
    """(counts[E], offsets[E+1], perm[valid pairs], n_invalid) of a stable expert sort."""
    ids = np.ascontiguousarray(ids, np.int32).ravel()
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    perm = np.zeros(max(ids.size, 1), np.int32)
    bad = lib().orc_route(_ptr(ids), ids.size, E, _ptr(counts), _ptr(offsets), _ptr(perm))
    return counts, offsets, perm[: ids.size - bad], int(bad)


def silu(g: np.ndarray) -> np.ndarray:
    """g * sigmoid(g) = g / (1 + exp(-g)) in float64 (exp overflow gives -0.0)."""
    g = np.asarray(g, np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu(gate_up: np.ndarray) -> np.ndarray:
    """SwiGLU expert activation: the last axis holds the gate rows [0, I)
    then the up rows [I, 2I); returns silu(gate) * up, shape [..., I]."""
    gu = np.asarray(gate_up, np.float64)
    I = gu.shape[-1] // 2
    return silu(gu[..., :I]) * gu[..., I:2 * I]


def combine(y_pairs: np.ndarray, route_w: np.ndarray) -> np.ndarray:
    """Router-weighted combine: y[t] = sum_j route_w[t, j] * y_pairs[t, j, :]
    (float64; a NaN in any slot makes the token's row NaN)."""
    yp = np.asarray(y_pairs, np.float64)
    w = np.asarray(route_w, np.float64)
    T, k = w.shape
    out = np.zeros((T, yp.shape[-1]), np.float64)
    for j in range(k):
        out += w[:, j:j + 1] * yp[:, j, :]
    return out
