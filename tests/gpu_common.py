"""Shared helpers of the GPU parity tests (inputs from ``synth``, expected
values from ``oracle`` only)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth

# accuracy bars: fp32-accumulated matvec 1e-3, bf16-weight GEMM 2e-2
TOL_GEMV = 1e-3
TOL_BF16 = 2e-2


def announce(msg: str) -> None:
    sys.stdout.write(f"\n[case] {msg}\n")
    sys.stdout.flush()


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values that are exactly bf16 (torch's RNE cast, CPU)."""
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).float().numpy()


def make_weights(fmt: int, E: int, out: int, n: int, seed: int):
    wire = synth.wire(fmt, E * out, n, seed)
    streams = oracle.pack(fmt, wire, E * out, n)
    return wire, streams


def rel_err_per_vector(y: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """||y - ref|| / ||ref|| over the last axis (one value per (t, j) pair)."""
    y = y.astype(np.float64)
    num = np.linalg.norm(y - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return num / np.maximum(den, 1e-300)


def half_ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Half the spacing of bfloat16 values at |v| (8 significand bits): the
    largest error of one round-to-nearest cast of a value of that binade."""
    a = np.abs(np.asarray(v, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def bf16_storage_excess(h: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per vector (last axis): (||h - ref|| - ||half-ulp of the cast||) / ||ref||
    for h stored as bfloat16 after a float32 computation of ref.  The cast
    adds at most half a bf16 spacing per element (taken at the larger of
    |h| and |ref|, so a value rounded into the next binade is covered), so
    the excess is at most the float32 computation's own relative error: an
    excess above the matvec's bar proves that error is above it.  (A plain relative error against the rounded or
    unrounded reference would charge a whole bf16 step to a vector whenever
    an element lies within the matvec's error of a rounding boundary.)"""
    h = np.asarray(h, np.float64)
    ref = np.asarray(ref, np.float64)
    allow = np.linalg.norm(half_ulp_bf16(np.maximum(np.abs(h), np.abs(ref))), axis=-1)
    return (np.linalg.norm(h - ref, axis=-1) - allow) / np.maximum(np.linalg.norm(ref, axis=-1), 1e-300)


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()
