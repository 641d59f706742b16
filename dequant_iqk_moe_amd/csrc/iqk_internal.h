// iqk_internal.h -- shared between the host entry points and the HIP kernels
// of the IQ_K routed-expert library.  Nothing here is part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/iqk.h"
#include "iqk_layout.h"

namespace iqk {

// Nonzero when a byte of w is not -1, 0 or +1 (0xFF, 0x00, 0x01), the
// values of the IQ1_S_R4 grid: those are the bytes whose bits 1..7 are all
// equal, except -2 (bits 1..7 set, bit 0 clear).
__device__ __forceinline__ uint32_t non_ternary(uint32_t w) {
    return ((w ^ (w >> 1)) & 0x7E7E7E7Eu) | (w & ~(w << 7) & 0x80808080u);
}


// Dequantization / producer launch description.
struct DequantLaunch {
    int fmt;
    int out_dtype;
    int64_t R, n, row0, nrows;
    const uint8_t* streams;
    Planes pl;
    float values[8];
    const int8_t* grid;
    void* out;
};

// Decode matvec launch description.
struct GemvLaunch {
    int fmt;
    int64_t E, out, n;
    const uint8_t* streams;
    Planes pl;
    uint32_t tab_lo, tab_hi;  // int8 table m_0..m_3 and m_4..m_7
    float tab_scale;          // 2^e with values[i] = m_i * 2^e
    const int8_t* grid;
    const void* x;
    int x_dtype, x_slots;
    const int32_t* ids;
    int64_t T;
    int k;
    float* y;
    uint32_t* sink;          // floor variant output (y unused)
    int mode;                // 0 plain y[T,k,out], 1 SwiGLU h[T,k,out/2] bf16, 2 combine y[T,out]
    uint16_t* h;             // mode 1
    const float* route_w;    // mode 2: [T, k]
};

struct RouteLaunch {
    const int32_t* ids;
    int64_t P, E;
    int sorted;  // 1: the caller states ids are non-decreasing (checked; the ranking is skipped when they are)
    int32_t *counts, *offsets, *perm;
    float* ynan = nullptr;  // if set: rows [P, yout] of the call's output, NaN for pairs with an invalid id
    int64_t yout = 0;
};

struct GemmLaunch {
    const void* W;
    int64_t E, out, n;
    const void* x;
    int x_slots;
    int64_t T;
    int k;
    const int32_t *offsets, *perm;
    float* y;
};

struct FusedLaunch {
    int fmt;
    int64_t E, out, n;
    const uint8_t* streams;
    Planes pl;
    const float* values;  // host float[8] (2-bit members)
    const int8_t* grid;   // device int8[2048 * 8] (IQ1_S_R4)
    const void* x;        // bf16 [T, x_slots, n]
    int x_slots, k;
    int64_t T;
    const int32_t *offsets, *perm;
    int64_t* plan;        // device int64[E + 1] (scratch: per-expert cost prefix)
    float* y;
};

hipError_t launch_dequant(const DequantLaunch& a, bool floor_variant, hipStream_t s);
hipError_t launch_fused_prefill(const FusedLaunch& a, hipStream_t s);
hipError_t launch_gemv(const GemvLaunch& a, bool floor_variant, hipStream_t s);
// grouped decode matvec (plain y): routing arrays from launch_route, plan =
// device int64[E + 1] scratch
hipError_t launch_gemv_grouped(const GemvLaunch& a, const int32_t* offsets, const int32_t* perm, int64_t* plan,
                               hipStream_t s);
hipError_t launch_route(const RouteLaunch& a, hipStream_t s);
hipError_t launch_grouped_gemm(const GemmLaunch& a, hipStream_t s);
hipError_t launch_swiglu(const float* y_gu, int64_t P, int64_t I, uint16_t* h, hipStream_t s);
hipError_t launch_combine(const float* y, const float* w, int64_t T, int k, int64_t out, float* yc, hipStream_t s);
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words, hipStream_t s);
hipError_t launch_stream_write(void* buf, size_t bytes, uint32_t value, int runs, hipStream_t s);

}  // namespace iqk
