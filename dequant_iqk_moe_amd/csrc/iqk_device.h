// iqk_device.h -- device-side access to the canonical per-row streams,
// shared by the decode matvec and the fused prefill (and the SwiGLU
// arithmetic shared by the matvec epilogue and the standalone glue kernel).
//
// "mlx-iqk" package description, "Format": per-row planes (qs, scl, sch,
// sex, dv for the 2-bit members; qs, qh, dv for IQ1_S_R4), here stored
// plane-major over the expert-stacked rows, each plane k-contiguous.  A
// lane reads the words of one 64-weight chunk of one row: one 16-byte code
// load (8 bytes for IQ1_S_R4) plus the small planes of that chunk.
#pragma once

#include "iqk_internal.h"

namespace iqk {

// silu(g) * u = g / (1 + exp(-g)) * u in float32, with the hardware
// exponential (v_exp_f32 of -g log2 e) and reciprocal (v_rcp_f32): about an
// ulp each, far below the bf16 rounding the SwiGLU output gets.  One
// definition for the matvec epilogue and the standalone kernel, so the two
// agree bit for bit.
__device__ __forceinline__ float silu_mul(float g, float u) {
    const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

__device__ __forceinline__ float half_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// Raw buffer resources.  An access at or past a resource's record count
// reads zero and a store there is dropped, so every row load and result
// store below is issued by every lane in every case: work that is absent (a
// row past the end, a group past the wave's last, an invalid expert id) gets
// an out-of-range offset or a resource of zero records instead of a branch.
// With no memory operation behind a branch the compiler counts outstanding
// loads exactly, and a wave waits for one group of rows while the next group
// stays in flight.
using Rsrc = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;  // raw (unswizzled) buffer, 32-bit data format
constexpr uint32_t kOob = 0x80000000u;  // an offset past every resource used here

__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
// Cache policy of a buffer load (its aux operand): the default, or the
// non-temporal hint for data a launch reads once.
constexpr int kCacheDefault = 0;
constexpr int kNonTemporal = 2;

template <int AUX = kCacheDefault>
__device__ __forceinline__ uint4 ld128(Rsrc r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX);
    return make_uint4(v[0], v[1], v[2], v[3]);
}
template <int AUX = kCacheDefault>
__device__ __forceinline__ uint2 ld64(Rsrc r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, AUX);
    return make_uint2(v[0], v[1]);
}
template <int AUX = kCacheDefault>
__device__ __forceinline__ uint32_t ld32(Rsrc r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, AUX); }
template <int AUX = kCacheDefault>
__device__ __forceinline__ uint32_t ld16(Rsrc r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, AUX); }
template <int AUX = kCacheDefault>
__device__ __forceinline__ uint32_t ld8(Rsrc r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, AUX); }

// Raw stream words of the 64 weights one lane owns in one row.
struct RowData {
    uint4 q;  // codes (IQ1_S_R4: q.x, q.y = low index bytes of 8 groups)
    uint32_t a, b, c, d;
};

// Byte strides of the planes per row.
template <int FMT, int N>
struct Strides {
    static constexpr int QS = FMT == IQK_IQ1_S_R4 ? N / 8 : N / 4;
    static constexpr int P1 = FMT == IQK_IQ2_K ? N / 32 : (FMT == IQK_IQ2_KS ? N / 64 : N / 16);
    static constexpr int P2 = FMT == IQK_IQ2_K ? N / 128 : (FMT == IQK_IQ2_KS ? N / 256 : 2);
    static constexpr int P3 = FMT == IQK_IQ2_K ? N / 128 : (FMT == IQK_IQ2_KS ? N / 256 : 0);
    static constexpr int P4 = FMT == IQK_IQ2_KS ? 2 : 0;
};

// Plane resources of one expert's rows; zero records for an invalid id, so
// its loads read zeros and move no data.
struct ExpertRes {
    Rsrc q, a, b, c, d;
    const uint8_t* dp;  // the expert's per-row scale plane (expert 0's for an invalid id)
    uint32_t dmax;      // its last row (reads of later rows are clamped to it)
};

template <int FMT, int N, class P>
__device__ __forceinline__ ExpertRes expert_res(const P& p, int e) {
    using St = Strides<FMT, N>;
    const bool valid = (unsigned)e < (unsigned)p.E;
    const int64_t row0 = (int64_t)(valid ? e : 0) * p.out;
    const uint32_t rows = valid ? (uint32_t)p.out : 0u;
    const uint8_t* S = p.S;
    ExpertRes r;
    r.dp = nullptr;  // (IQ2_K has no per-row scale)
    r.dmax = (uint32_t)p.out - 1u;
    r.q = make_rsrc(S + p.off0 + row0 * St::QS, rows * St::QS);
    r.a = make_rsrc(S + p.off1 + row0 * St::P1, rows * St::P1);
    if constexpr (FMT == IQK_IQ2_K) {
        r.b = make_rsrc(S + p.off2 + row0 * St::P2, rows * St::P2);
        r.d = make_rsrc(S + p.off3 + row0 * St::P3, rows * St::P3);
        r.c = r.b;
    } else if constexpr (FMT == IQK_IQ2_KS) {
        r.b = make_rsrc(S + p.off2 + row0 * St::P2, rows * St::P2);
        r.c = make_rsrc(S + p.off3 + row0 * St::P3, rows * St::P3);
        r.d = make_rsrc(S + p.off4 + row0 * 2, rows * 2u);
        r.dp = S + p.off4 + row0 * 2;
    } else {
        r.d = make_rsrc(S + p.off2 + row0 * 2, rows * 2u);
        r.dp = S + p.off2 + row0 * 2;
        r.b = r.c = r.d;
    }
    return r;
}

// 16-bit word at a wave-uniform address, through the scalar data cache (the
// constant address space makes it a scalar load).  The load takes the aligned
// 32-bit word holding it: that word lies in the same page as the 16-bit word,
// so it stays in mapped memory even at the end of a buffer.
__device__ __forceinline__ uint32_t sload_u16(const uint8_t* p) {
    const uintptr_t a = (uintptr_t)p;
    const __attribute__((address_space(4))) uint32_t* cp =
        (const __attribute__((address_space(4))) uint32_t*)(a & ~(uintptr_t)3);
    const uint32_t w = *cp;
    return (a & 2u) ? (w >> 16) : (w & 0xFFFFu);
}

// The words one lane needs for expert row `row` (rows at or past `out` are
// out of range and read zeros).  Resources are uniform, offsets per lane;
// AUX is the loads' cache policy.
template <int FMT, int N, int AUX = kCacheDefault, bool NO_D = false>
__device__ __forceinline__ RowData load_row(const ExpertRes& x, uint32_t row, uint32_t c) {
    using St = Strides<FMT, N>;
    RowData r;
    if constexpr (FMT == IQK_IQ2_K) {
        r.q = ld128<AUX>(x.q, row * St::QS + 16u * c);
        r.a = ld16<AUX>(x.a, row * St::P1 + 2u * c);
        r.b = ld8<AUX>(x.b, row * St::P2 + (c >> 1));
        r.c = 0;
        r.d = ld16<AUX>(x.d, row * St::P3 + 2u * (c >> 2));
    } else if constexpr (FMT == IQK_IQ2_KS) {
        r.q = ld128<AUX>(x.q, row * St::QS + 16u * c);
        r.a = ld8<AUX>(x.a, row * St::P1 + c);
        r.b = ld8<AUX>(x.b, row * St::P2 + (c >> 2));
        r.c = ld8<AUX>(x.c, row * St::P3 + (c >> 2));
        r.d = NO_D ? 0u : ld16<AUX>(x.d, row * 2u);
    } else {
        const uint2 qq = ld64<AUX>(x.q, row * St::QS + 8u * c);
        r.q = make_uint4(qq.x, qq.y, 0, 0);
        r.a = ld32<AUX>(x.a, row * St::P1 + 4u * c);
        r.b = 0;
        r.c = 0;
        r.d = NO_D ? 0u : ld16<AUX>(x.d, row * 2u);
    }
    return r;
}

}  // namespace iqk
