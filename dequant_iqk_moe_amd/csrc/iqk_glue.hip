// iqk_glue.hip -- the MoE layer steps either side of the routed projections,
// as standalone kernels for the prefill paths (the decode matvec has them as
// epilogues).
//
// "mlx-iqk" package description, "Surface": the routed projection is a
// switch-linear call y[T, k, out] = proj(x, indices); a SwiGLU expert feeds
// silu(gate) * up of its gate/up projection to down, and the layer output is
// the router-weighted sum of the k slots.  The arithmetic is the decode
// epilogues': h = g / (1 + exp(-g)) * u in float32 (silu_mul), one
// round-to-nearest-even cast to bf16; y[t] = sum_j (w[t, j] * y[t, j]) with each product rounded
// once and the sum taken in slot order.  Both are HBM-bound elementwise
// passes (16-byte loads, grid-stride).
#include "iqk_device.h"

namespace iqk {
namespace {

constexpr int kGlueThreads = 256;

__device__ __forceinline__ uint32_t glue_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;  // NaN stays a quiet NaN
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// y_gu [P, 2I] (gate columns [0, I), up columns [I, 2I)) -> h [P, I] bf16;
// one thread per 4 consecutive h values (I % 4 == 0)
__global__ __launch_bounds__(kGlueThreads) void swiglu_kernel(const float* __restrict__ y_gu, int64_t P, int64_t I,
                                                              uint16_t* __restrict__ h) {
    const int64_t q = I / 4;
    const int64_t total = P * q;
    for (int64_t i = (int64_t)blockIdx.x * kGlueThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kGlueThreads) {
        const int64_t p = i / q;
        const int64_t c = (i - p * q) * 4;
        const float4 g = *(const float4*)(y_gu + p * 2 * I + c);
        const float4 u = *(const float4*)(y_gu + p * 2 * I + I + c);
        const float gv[4] = {g.x, g.y, g.z, g.w};
        const float uv[4] = {u.x, u.y, u.z, u.w};
        uint32_t o[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = glue_bf16(silu_mul(gv[j], uv[j]));
        *(uint2*)(h + p * I + c) = make_uint2(o[0] | (o[1] << 16), o[2] | (o[3] << 16));
    }
}

// y [T, k, out], w [T, k] -> yc [T, out]; one thread per 4 consecutive
// outputs (out % 4 == 0)
__global__ __launch_bounds__(kGlueThreads) void combine_kernel(const float* __restrict__ y,
                                                               const float* __restrict__ w, int64_t T, int k,
                                                               int64_t out, float* __restrict__ yc) {
    const int64_t q = out / 4;
    const int64_t total = T * q;
    for (int64_t i = (int64_t)blockIdx.x * kGlueThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kGlueThreads) {
        const int64_t t = i / q;
        const int64_t c = (i - t * q) * 4;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j = 0; j < k; ++j) {
            const float wj = w[t * k + j];
            const float4 v = *(const float4*)(y + (t * k + j) * out + c);
            // product rounded on its own, then added in slot order (no fusion)
            const float4 pr = make_float4(__fmul_rn(wj, v.x), __fmul_rn(wj, v.y), __fmul_rn(wj, v.z),
                                          __fmul_rn(wj, v.w));
            if (j == 0) {
                acc = pr;
            } else {
                acc.x = __fadd_rn(acc.x, pr.x);
                acc.y = __fadd_rn(acc.y, pr.y);
                acc.z = __fadd_rn(acc.z, pr.z);
                acc.w = __fadd_rn(acc.w, pr.w);
            }
        }
        *(float4*)(yc + t * out + c) = acc;
    }
}

unsigned glue_blocks(int64_t items) {
    int64_t b = (items + kGlueThreads - 1) / kGlueThreads;
    b = b < 1 ? 1 : (b > 256 * 8 ? 256 * 8 : b);
    return (unsigned)b;
}

}  // namespace

hipError_t launch_swiglu(const float* y_gu, int64_t P, int64_t I, uint16_t* h, hipStream_t s) {
    hipLaunchKernelGGL(swiglu_kernel, dim3(glue_blocks(P * (I / 4))), dim3(kGlueThreads), 0, s, y_gu, P, I, h);
    return hipGetLastError();
}

hipError_t launch_combine(const float* y, const float* w, int64_t T, int k, int64_t out, float* yc, hipStream_t s) {
    hipLaunchKernelGGL(combine_kernel, dim3(glue_blocks(T * (out / 4))), dim3(kGlueThreads), 0, s, y, w, T, k, out,
                       yc);
    return hipGetLastError();
}

}  // namespace iqk
