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


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()
