"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds none of the method's arithmetic: it draws random bytes,
places fp16 scale values where the stand-in wire layouts keep them, and draws
activations, value tables, ternary grids and expert ids.  Both the oracle and
the GPU path consume exactly the arrays returned here.

Workload shapes follow the "mlx-iqk" package description (routed geometry in
its introduction: 256 experts, six selected, gate/up 2048x4096, down
4096x2048) and the synthetic recipes of the five benchmark configurations:
scales |N(0,1)|*0.01 stored as fp16, codes / scale indices / alphabet bits
uniform (uniform random bytes give exactly that), uniform top-6 routing
without replacement, activations N(0,1).
"""
from __future__ import annotations

import numpy as np

IQ2_KS, IQ2_K, IQ1_S_R4 = 1, 2, 3

# bytes per row of each member, per the "Format" section budgets
def row_bytes(fmt: int, n: int) -> int:
    if fmt == IQ2_KS:
        return 2 + 70 * n // 256
    if fmt == IQ2_K:
        return 76 * n // 256
    if fmt == IQ1_S_R4:
        return 2 + 6 * n // 32
    raise ValueError(fmt)


def _rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def _scales(rng: np.random.Generator, count: int, sigma: float) -> np.ndarray:
    """fp16 bit patterns of |N(0,1)| * sigma (numpy's float16 cast)."""
    v = np.abs(rng.standard_normal(count)) * sigma
    return v.astype(np.float16).view(np.uint16)


def random_bytes(nbytes: int, seed: int) -> np.ndarray:
    return np.frombuffer(_rng(seed).bytes(nbytes), np.uint8).copy()


def wire(fmt: int, rows: int, n: int, seed: int, sigma: float = 0.01) -> np.ndarray:
    """Stand-in ik wire bytes for a [rows, n] tensor: every byte uniform random
    (so codes, scale indices, alphabet / sign bits, grid indices and ls are
    uniform over their ranges) except the fp16 scales, which are drawn as
    |N(0,1)| * sigma.  Scale positions: IQ2_KS one fp16 at the start of each
    row; IQ2_K one fp16 at the start of each 76-byte block; IQ1_S_R4 four
    fp16 at the start of each four-row group."""
    rb = row_bytes(fmt, n)
    rng = _rng(seed)
    w = np.frombuffer(rng.bytes(rows * rb), np.uint8).copy()
    if fmt == IQ2_KS:
        v = w.reshape(rows, rb)
        v[:, 0:2] = _scales(rng, rows, sigma).view(np.uint8).reshape(rows, 2)
    elif fmt == IQ2_K:
        nb = rows * n // 256
        v = w.reshape(nb, 76)
        v[:, 0:2] = _scales(rng, nb, sigma).view(np.uint8).reshape(nb, 2)
    elif fmt == IQ1_S_R4:
        if rows % 4:
            raise ValueError("IQ1_S_R4 wire comes in groups of four rows")
        g = rows // 4
        v = w.reshape(g, 4 * rb)
        v[:, 0:8] = _scales(rng, 4 * g, sigma).view(np.uint8).reshape(g, 8)
    else:
        raise ValueError(fmt)
    return w


def _scale_mask(fmt: int, rows: int, n: int) -> np.ndarray:
    """bool [rows * row_bytes]: the bytes that hold fp16 scales in the wire"""
    rb = row_bytes(fmt, n)
    m = np.zeros(rows * rb, bool)
    if fmt == IQ2_KS:
        v = m.reshape(rows, rb)
        v[:, 0:2] = True
    elif fmt == IQ2_K:
        v = m.reshape(rows * n // 256, 76)
        v[:, 0:2] = True
    else:
        v = m.reshape(rows // 4, 4 * rb)
        v[:, 0:8] = True
    return m


def wire_experts(fmt: int, E: int, out: int, n: int, seed: int, sigma: float = 0.01) -> np.ndarray:
    """Stand-in wire of E stacked [out, n] experts built cheaply at full size:
    one expert drawn as `wire`, and expert e a copy whose non-scale bytes are
    XORed with a byte of its own (every expert distinct, bytes still uniform,
    scales unchanged)."""
    base = wire(fmt, out, n, seed, sigma)
    keep = _scale_mask(fmt, out, n)
    pat = np.where(keep, 0, 1).astype(np.uint8)
    salt = _rng(seed + 1).integers(1, 256, size=E).astype(np.uint8)
    salt[0] = 0
    w = np.empty((E, base.size), np.uint8)
    for e in range(E):
        np.bitwise_xor(base, pat * salt[e], out=w[e])
    return w.reshape(-1)


def values_table(seed: int) -> np.ndarray:
    """Eight integers in [-32, 31] as float32: a stand-in for the 8-entry
    value table (two 4-entry alphabets), exact in fp16 and bf16."""
    return _rng(seed).integers(-32, 32, size=8).astype(np.float32)


def ternary_grid(seed: int) -> np.ndarray:
    """2048 x 8 int8 grid of i.i.d. uniform values in {-1, 0, 1}."""
    return _rng(seed).integers(-1, 2, size=(2048, 8)).astype(np.int8)


def topk_ids(T: int, k: int, E: int, seed: int) -> np.ndarray:
    """[T, k] int32 expert ids, each token's k ids uniform without replacement."""
    rng = _rng(seed)
    out = np.empty((T, k), np.int32)
    for t in range(T):
        out[t] = rng.choice(E, size=k, replace=False)
    return out


def normal(shape, seed: int) -> np.ndarray:
    """float32 N(0,1) samples (cast to bf16 by the caller where needed)."""
    return _rng(seed).standard_normal(shape).astype(np.float32)
