"""The Python binding refuses a device buffer of the wrong size before any
library call (no GPU needed).

The kernels write or read exactly T*k*out outputs, nrows*in dequantized
values, 2048*8 grid bytes and so on; a shorter buffer would be overrun on
the device.  The checks run on the tensors' metadata, so a stand-in object
with the attributes of a contiguous device tensor is enough here: every call
below raises IqkValueError(E_SIZE) while evaluating its arguments, before
the library sees a pointer.
"""
import numpy as np
import pytest
import torch

import dequant_iqk_moe_amd as q

E_SIZE = -6


class FakeDev:
    """metadata of a contiguous device tensor (never dereferenced)"""

    def __init__(self, shape, dtype):
        self.shape = tuple(shape)
        self.dtype = dtype
        self.is_cuda = True
        self.device = "cuda"

    def numel(self):
        return int(np.prod(self.shape)) if self.shape else 1

    def dim(self):
        return len(self.shape)

    def element_size(self):
        return torch.empty((), dtype=self.dtype).element_size()

    def is_contiguous(self):
        return True

    def data_ptr(self):
        return 0x1000


FMT, E, OUT, N, T, K = q.IQ2_K, 8, 64, 512, 3, 4
VALUES = np.arange(8, dtype=np.float32)


def _w(fmt=FMT, out=OUT):
    return q.Weights(fmt, E, out, N, FakeDev((E * out * q.row_bytes(fmt, N),), torch.uint8))


def _x(slots=1):
    return FakeDev((T, slots, N), torch.bfloat16)


def _ids():
    return FakeDev((T, K), torch.int32)


def f32(*shape):
    return FakeDev(shape, torch.float32)


def _refused(fn):
    with pytest.raises(q.IqkValueError) as ei:
        fn()
    assert ei.value.code == E_SIZE, str(ei.value)


SHORT = 1  # elements missing from the undersized buffers


def test_matvec_family_refuses_short_outputs():
    w = _w()
    _refused(lambda: q.moe_gemv(w, _x(), _ids(), VALUES, y=f32(T * K * OUT - SHORT)))
    _refused(lambda: q.moe_gemv_swiglu(w, _x(), _ids(), VALUES,
                                       h=FakeDev((T * K * OUT // 2 - SHORT,), torch.bfloat16)))
    _refused(lambda: q.moe_gemv_combine(w, _x(K), _ids(), f32(T, K), VALUES, y=f32(T * OUT - SHORT)))
    _refused(lambda: q.moe_gemv_combine(w, _x(K), _ids(), f32(T * K - SHORT), VALUES, y=f32(T, OUT)))
    ws = FakeDev((1 << 20,), torch.uint8)
    _refused(lambda: q.moe_gemv_grouped(w, _x(), _ids(), VALUES, workspace=ws, y=f32(T * K * OUT - SHORT)))
    _refused(lambda: q.moe_auto(w, _x(), _ids(), VALUES, workspace=ws, y=f32(T * K * OUT - SHORT)))
    _refused(lambda: q.floor_gemv(w, _x(), _ids(), VALUES, sink=FakeDev((T * K * OUT - SHORT,), torch.int32)))
    # the activation and the grid
    _refused(lambda: q.moe_gemv(w, FakeDev((T, 1, N - 1), torch.bfloat16), _ids(), VALUES, y=f32(T, K, OUT)))
    w4 = _w(q.IQ1_S_R4)
    _refused(lambda: q.moe_gemv(w4, _x(), _ids(), None, FakeDev((2048 * 8 - SHORT,), torch.int8), y=f32(T, K, OUT)))


def test_producer_and_prefill_refuse_short_buffers():
    w = _w()
    _refused(lambda: q.dequant(w, VALUES, None, out=FakeDev((E * OUT * N - SHORT,), torch.bfloat16)))
    _refused(lambda: q.dequant(w, VALUES, None, row0=3, nrows=5, out=FakeDev((5, N - 1), torch.float32)))
    _refused(lambda: q.floor_dequant(w, out=FakeDev((E * OUT, N - 1), torch.bfloat16)))
    w4 = _w(q.IQ1_S_R4)
    _refused(lambda: q.dequant(w4, None, FakeDev((100,), torch.int8), out=FakeDev((E * OUT, N), torch.bfloat16)))
    ws = FakeDev((1 << 30,), torch.uint8)
    _refused(lambda: q.moe_prefill(w, _x(), _ids(), VALUES, workspace=ws, y=f32(T * K * OUT - SHORT)))
    _refused(lambda: q.moe_prefill_fused(w, _x(), _ids(), VALUES, workspace=ws, y=f32(T * K * OUT - SHORT)))


def test_glue_and_gemm_refuse_short_buffers():
    I = 32
    _refused(lambda: q.swiglu(f32(5, 2 * I), h=FakeDev((5 * I - SHORT,), torch.bfloat16)))
    _refused(lambda: q.combine(f32(T, K, OUT), f32(T, K), yc=f32(T * OUT - SHORT)))
    _refused(lambda: q.combine(f32(T, K, OUT), f32(T * K - SHORT), yc=f32(T, OUT)))
    W = FakeDev((E, OUT, N), torch.bfloat16)
    x = FakeDev((T, 1, N), torch.bfloat16)
    offs, perm = FakeDev((E + 1,), torch.int32), FakeDev((T * K,), torch.int32)
    _refused(lambda: q.grouped_gemm(W, x, T, K, offs, perm, y=f32(T * K * OUT - SHORT)))
    _refused(lambda: q.grouped_gemm(W, x, T, K, FakeDev((E,), torch.int32), perm, y=f32(T, K, OUT)))
    _refused(lambda: q.grouped_gemm(W, x, T, K, offs, FakeDev((T * K - SHORT,), torch.int32), y=f32(T, K, OUT)))
