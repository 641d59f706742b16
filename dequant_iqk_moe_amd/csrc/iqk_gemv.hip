// iqk_gemv.hip -- fused dequantize-and-matvec for routed-expert decode.
//
// "mlx-iqk" package description:
//   - "Surface": a call with few token-expert pairs runs a fused decode
//     matvec; one pass over the reduction axis per instance, so only
//     instantiated input widths are accepted;
//   - introduction: codes are read from one contiguous 2-bit plane, the
//     8-entry value table is held in a narrow type and each sub-block's
//     alphabet is taken once per sub-block, not once per weight;
//   - "Format": the stream tables and the two reconstruction formulas.
//
// gfx950 design.  The matvec is bound by HBM bytes, but at 8 TB/s the
// vector ALUs have only ~1.3-1.5 lane-instructions per weight, so the decode
// is integer and 4-wide:
//   * each lane owns 64 consecutive k of a row (one 16-byte load of the code
//     plane); a wave covers 4096 k per load instruction (1 row at in=4096,
//     2 rows at 2048, 8 rows at 512), every load coalesced along k;
//   * the activation is converted once per workgroup to 15-bit fixed point
//     per 64-value block (scale 2^(13 - emax)), split into two int8 planes
//     (hi, lo) in LDS, then held by each lane in 32 VGPRs for all its rows;
//   * 2-bit members: (q >> 2j) & 0x03030303 spreads four codes into four
//     bytes, OR-ing 4 * alphabet makes each byte an index into the 8-entry
//     int8 table, and one v_perm_b32 looks up four weights; v_dot4_i32_i8
//     against the hi and lo planes accumulates exact int32 per sub-block,
//     v_mad_i32_i24 applies the signed scale index.  The fixed-point x is
//     pre-permuted in LDS to match the spread order, so no weight moves;
//   * IQ1_S_R4: the 2048 x 8 int8 grid is staged in LDS (16 KiB); each
//     8-weight group is one ds_read_b64 and four v_dot4_i32_i8, the +-1/8
//     shift is applied through the block sum of x;
//   * per-lane partials of 4 rows are reduced with v_permlane32_swap,
//     v_permlane16_swap and DPP (10 instructions per 4 rows).
// Latency: a decode launch is a few microseconds long.  The activation is
// read and converted first (row loads issued before it would queue ahead of
// it), the workgroup barrier waits only for LDS traffic, every wave then
// requests its first two row groups at once and each later group two groups
// ahead.  One large workgroup per CU (up to 16 waves) amortizes the
// activation conversion over ~100 rows; a launch small enough for two
// workgroups of at most 8 waves each per CU runs two, so one block's
// start-up overlaps the other's decode.  Rows of a workgroup are
// contiguous, so the small per-row planes share cache lines.
//
// The grouped matvec at the end of this file serves a few tokens per
// expert: after the routing gather, one pass over each selected expert's
// rows decodes every chunk once into int8 weight words and multiplies it
// with all of the expert's tokens, whose activations each lane converts
// into its own registers (a lane's chunk of k is the same for every row).
#include "iqk_device.h"

namespace iqk {
namespace {

#ifndef IQK_GEMV_TARGET_BLOCKS
#define IQK_GEMV_TARGET_BLOCKS 256  // workgroups per launch (one per CU; two for small launches)
#endif
#ifndef IQK_GEMV_MIN_GROUPS
#define IQK_GEMV_MIN_GROUPS 2       // reduction groups per wave when the block has >= 8
#endif
#ifndef IQK_GEMV_MAX_WAVES
#define IQK_GEMV_MAX_WAVES 16        // waves per workgroup (launch bound)
#endif
constexpr int kMaxWaves = IQK_GEMV_MAX_WAVES;

// Unsigned division by a launch constant d >= 1 without a division sequence
// (the scalar unit has no divide; the compiler's expansion is ~40
// instructions on the kernel's critical path).  Round-up method: with
// l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1 and t = mulhi(n, m),
// n / d = (t + ((n - t) >> 1)) >> (l - 1) for every 32-bit n and d >= 2
// (T. Granlund and P. L. Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994); d = 1 is passed through.
struct FastDiv {
    uint32_t m, s, d;
};

inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f{0u, 0u, d};
    if (d > 1) {
        uint32_t l = 0;
        while ((1ull << l) < d) ++l;
        f.m = (uint32_t)((((1ull << 32) * ((1ull << l) - d)) / d) + 1);
        f.s = l - 1;
    }
    return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
    if (f.d == 1) return n;
    const uint32_t t = __umulhi(n, f.m);
    return (t + ((n - t) >> 1)) >> f.s;
}

// What a launch writes after the row sums (see the entry points):
//   kPlain   y[t, j, o] (fp32), one unit = one pair's row group;
//   kSwiGLU  h[t, j, i] = silu(gate_i) * up_i (bf16) from a gate/up tensor
//            whose rows [0, I) are gate and [I, 2I) up; a unit holds
//            RPG/2 gate rows and the matching up rows;
//   kCombine y[t, o] = sum_j w[t, j] * (row o of expert ids[t, j]) . x_j
//            (fp32); a unit is one token's row group, visited once per slot
//            j = 0..k-1 in order, accumulated in registers.
enum GemvMode { kPlain = 0, kSwiGLU = 1, kCombine = 2 };

struct GemvParams {
    const uint8_t* S;
    int64_t off0, off1, off2, off3, off4;
    int32_t E, out;
    uint32_t tab_lo, tab_hi;
    float tab_scale;
    const int8_t* grid;
    const void* x;
    int32_t x_slots, k;
    const int32_t* ids;
    float* y;           // kPlain: [T, k, out]; kCombine: [T, out]
    uint32_t* sink;     // floor variant output
    uint16_t* h;        // kSwiGLU: bf16 [T, k, out / 2]
    const float* rw;    // kCombine: router weights [T, k]
    int32_t outers;     // pairs (kPlain, kSwiGLU) or tokens (kCombine)
    int32_t upo;        // units per outer
    int32_t ubase;      // units per block: ubase, plus one for the first urem blocks
    int32_t urem;       //   (kCombine: per block of one token, bpt blocks per token)
    int32_t bpt;
    FastDiv dupo, dk, dbpt;
};

template <int N>
struct Geo {
    static constexpr int LPR = N / 64;                                // lanes per row
    static constexpr int RPI = 64 / LPR;                              // rows per wave iteration
    static constexpr int GIT = LPR == 64 ? 4 : (LPR == 32 ? 2 : 1);   // iterations per reduction group
    static constexpr int RPG = GIT * RPI;                             // rows per reduction group
};


// Workgroup barrier for LDS only: global loads issued before it stay in
// flight (a full __syncthreads would wait for them).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) { return __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) { return __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ uint32_t dpp_half_mirror(uint32_t v) { return __builtin_amdgcn_update_dpp(0u, v, 0x141, 0xF, 0xF, false); }
__device__ __forceinline__ uint32_t dpp_mirror(uint32_t v) { return __builtin_amdgcn_update_dpp(0u, v, 0x140, 0xF, 0xF, false); }

// Addition on the carried 32-bit values: float for results, integer for the
// floor variant's accumulator.
template <bool INT>
__device__ __forceinline__ uint32_t add32(uint32_t a, uint32_t b) {
    if constexpr (INT) return a + b;
    else return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
}

// Sum within each 16-lane row (xor 1, xor 2, half-mirror, mirror): every
// lane of the row ends with the row's total.
template <bool INT>
__device__ __forceinline__ uint32_t reduce16(uint32_t v) {
    v = add32<INT>(v, dpp_xor1(v));
    v = add32<INT>(v, dpp_xor2(v));
    v = add32<INT>(v, dpp_half_mirror(v));
    v = add32<INT>(v, dpp_mirror(v));
    return v;
}

template <bool INT>
__device__ __forceinline__ uint32_t reduce8(uint32_t v) {
    v = add32<INT>(v, dpp_xor1(v));
    v = add32<INT>(v, dpp_xor2(v));
    v = add32<INT>(v, dpp_half_mirror(v));
    return v;
}

// Reduce the GIT per-lane partials of one reduction group.  Returns the sum
// for the row this lane reports (row index within the group in *row_out),
// and whether this lane writes it.
template <int N, bool INT>
__device__ __forceinline__ uint32_t reduce_group(const uint32_t* part, int lane, int* row_out, bool* writer) {
    using G = Geo<N>;
    if constexpr (G::LPR == 64) {
        // part[i] = row i (all 64 lanes).  32-swap: rows {0,2} and {1,3}
        auto a = __builtin_amdgcn_permlane32_swap(part[0], part[2], false, false);
        auto b = __builtin_amdgcn_permlane32_swap(part[1], part[3], false, false);
        uint32_t u = add32<INT>(a[0], a[1]);  // lanes 0-31: row 0, lanes 32-63: row 2
        uint32_t v = add32<INT>(b[0], b[1]);  // lanes 0-31: row 1, lanes 32-63: row 3
        auto c = __builtin_amdgcn_permlane16_swap(u, v, false, false);
        uint32_t w = add32<INT>(c[0], c[1]);  // 16-lane row g holds row g
        w = reduce16<INT>(w);
        *row_out = lane >> 4;
        *writer = (lane & 15) == 0;
        return w;
    } else if constexpr (G::LPR == 32) {
        // part[i]: lanes 0-31 row 2i, lanes 32-63 row 2i+1
        auto c = __builtin_amdgcn_permlane16_swap(part[0], part[1], false, false);
        uint32_t w = add32<INT>(c[0], c[1]);  // 16-lane rows 0..3 hold rows 0, 2, 1, 3
        w = reduce16<INT>(w);
        const int g = lane >> 4;
        *row_out = ((g & 1) << 1) | (g >> 1);
        *writer = (lane & 15) == 0;
        return w;
    } else {
        // LPR == 8: part[0] lane l belongs to row l / 8
        uint32_t w = reduce8<INT>(part[0]);
        *row_out = lane >> 3;
        *writer = (lane & 7) == 0;
        return w;
    }
}

// Activation in LDS: per 64-value chunk, 64 hi bytes and 64 lo bytes in the
// order the decode consumes them, plus the chunk scale (and for IQ1_S_R4 the
// sums of the fixed-point values over each 32-weight block).
template <int N>
struct XLds {
    uint32_t hi[N / 4];
    uint32_t lo[N / 4];
    float scale[N / 64];
    int32_t bsum[N / 32];
};

// 16-byte slot of block i (0..3) of 64-value chunk c in an XLds plane.  The
// decode reads block i of chunk c = lane in one ds_read_b128 per wave;
// rotating the four blocks of a chunk by c / 4 puts the eight lanes served
// in one LDS cycle (chunks c and c + 4 would otherwise share banks) on
// distinct banks.
__device__ __forceinline__ int xslot(int c, int i) { return 4 * c + ((i + (c >> 2)) & 3); }

// Two 16-bit lanes added without a carry between them (v_pk_add_u16).
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t add_u16x2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, a) + __builtin_bit_cast(u16x2, b));
}

// Raw activation words of one 16-value block (bf16: 8 words, f32: 16).
template <int XDT>
struct XRaw {
    uint32_t w[XDT == IQK_BF16 ? 8 : 16];
};

template <int N, int XDT>
__device__ __forceinline__ XRaw<XDT> load_xblock(const void* xrow, int b) {
    XRaw<XDT> r;
    if constexpr (XDT == IQK_BF16) {
        const uint4* src = (const uint4*)xrow + 2 * b;
        const uint4 a = src[0], c = src[1];
        r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
        r.w[4] = c.x; r.w[5] = c.y; r.w[6] = c.z; r.w[7] = c.w;
    } else {
        const uint4* src = (const uint4*)xrow + 4 * b;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 f = src[i];
            r.w[4 * i] = f.x; r.w[4 * i + 1] = f.y; r.w[4 * i + 2] = f.z; r.w[4 * i + 3] = f.w;
        }
    }
    return r;
}

// Convert one 16-value block of the activation (block index b; the four
// blocks of a 64-value chunk sit in four consecutive lanes).
template <int FMT, int N, int XDT>
__device__ __forceinline__ void prep_block(const XRaw<XDT>& raw, XLds<N>& L, int b) {
    float v[16];
    if constexpr (XDT == IQK_BF16) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = __uint_as_float(raw.w[i] << 16);
            v[2 * i + 1] = __uint_as_float(raw.w[i] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = __uint_as_float(raw.w[i]);
    }
    float am = 0.f;  // (v_max3_f32 with |.| source modifiers)
#pragma unroll
    for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(v[i]));
    // the chunk's four blocks sit in one quad of lanes, all active together
    // (DPP within the quad, no LDS round trip); non-negative floats order as
    // their bit patterns
    uint32_t amax = __float_as_uint(am);
    amax = max(amax, dpp_xor1(amax));
    amax = max(amax, dpp_xor2(amax));
    int emax = (int)(amax >> 23) - 127;
    emax = emax < -100 ? -100 : emax;
    const float s = __builtin_ldexpf(1.0f, 13 - emax);
    // q = rint(v s), |q| <= 2^14, as one v_fma_f32: v s + 1.5 2^23 lands in
    // [2^23, 2^24), where float32 steps are 1, and rounds once to the
    // nearest integer, ties to even as rint (the added constant is even);
    // the word is then 0x4B400000 + q, whose low 16 bits are q's.
    uint32_t q[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) q[i] = __float_as_uint(__builtin_fmaf(v[i], s, 12582912.0f));
    // q = 256 hi + lo with lo in [-128, 127]: lo is q's low byte and hi the
    // second byte of q + 128 (16-bit), so each plane word is byte gathers
    // (v_perm_b32) of q packed two to a word, plus one packed 16-bit add.
    uint32_t wh[4], wl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        // 2-bit members: word j = values j, 4+j, 8+j, 12+j (the code-spread order);
        // IQ1_S_R4: natural order
        const int i0 = FMT == IQK_IQ1_S_R4 ? 4 * j : j;
        const int st = FMT == IQK_IQ1_S_R4 ? 1 : 4;
        const uint32_t w01 = __builtin_amdgcn_perm(q[i0 + st], q[i0], 0x05040100u);
        const uint32_t w23 = __builtin_amdgcn_perm(q[i0 + 3 * st], q[i0 + 2 * st], 0x05040100u);
        wl[j] = __builtin_amdgcn_perm(w23, w01, 0x06040200u);
        wh[j] = __builtin_amdgcn_perm(add_u16x2(w23, 0x00800080u), add_u16x2(w01, 0x00800080u), 0x07050301u);
    }
    const int slot = xslot(b >> 2, b & 3);
    *(uint4*)&L.hi[4 * slot] = make_uint4(wh[0], wh[1], wh[2], wh[3]);
    *(uint4*)&L.lo[4 * slot] = make_uint4(wl[0], wl[1], wl[2], wl[3]);
    if ((b & 3) == 0) L.scale[b >> 2] = __builtin_ldexpf(1.0f, emax - 13);
    if constexpr (FMT == IQK_IQ1_S_R4) {
        uint32_t sum = 0u - 16u * 0x4B400000u;  // (wrapping) sum of the q
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += q[i];
        sum += dpp_xor1(sum);
        if ((b & 1) == 0) L.bsum[b >> 1] = sum;
    }
}

// d = dot4(a, b) with the accumulator starting at zero (VOP3P form with an
// inline zero instead of a v_mov plus v_dot4c).
__device__ __forceinline__ int dot4_first(uint32_t a, uint32_t b) {
    int d;
    asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(d) : "v"(a), "v"(b));
    return d;
}

// (a & b) | c, left to the compiler (measured faster in context than a
// hand-placed v_bitop3_b32).
__device__ __forceinline__ uint32_t and_or_fast(uint32_t a, uint32_t b, uint32_t c) { return (a & b) | c; }

// int8 weights of two code words (16 each) from the value table: word i,
// byte b of w[i][jj] holds weight 4 b + jj, alphabet bits m[i] (0 or 4 in
// every byte).  The codes of a shift step come from one 64-bit shift of the
// word pair (v_lshrrev_b64 moves both words; the bits crossing from the
// high word into the low one land above each byte's two code bits, which
// the mask drops): 3 shifts per 32 weights instead of 6.
__device__ __forceinline__ void expand_pair(uint32_t q0, uint32_t q1, uint32_t m0, uint32_t m1, uint32_t tlo,
                                            uint32_t thi, uint32_t (&w0)[4], uint32_t (&w1)[4]) {
    const uint64_t qq = ((uint64_t)q1 << 32) | q0;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
        uint64_t sh = qq;
        if (jj > 0) asm("v_lshrrev_b64 %0, %1, %2" : "=v"(sh) : "i"(2 * jj), "v"(qq));
        w0[jj] = __builtin_amdgcn_perm(thi, tlo, and_or_fast((uint32_t)sh, 0x03030303u, m0));
        w1[jj] = __builtin_amdgcn_perm(thi, tlo, and_or_fast((uint32_t)(sh >> 32), 0x03030303u, m1));
    }
}

// 16 weights (4 words) against 4 activation words, as one chain.
template <bool FIRST>
__device__ __forceinline__ int dot16w(const uint32_t (&w)[4], const uint32_t* x4, int acc) {
    if constexpr (FIRST) acc = dot4_first(w[0], x4[0]);
    else acc = __builtin_amdgcn_sdot4((int)w[0], (int)x4[0], acc, false);
    acc = __builtin_amdgcn_sdot4((int)w[1], (int)x4[1], acc, false);
    acc = __builtin_amdgcn_sdot4((int)w[2], (int)x4[2], acc, false);
    acc = __builtin_amdgcn_sdot4((int)w[3], (int)x4[3], acc, false);
    return acc;
}

// Dot of one lane's 64 weights with its 64 fixed-point activations, before
// the per-lane float scale (fp16 d * chunk scale * table scale).
template <int FMT>
__device__ __forceinline__ float row_dot(const RowData& r, int c, const uint32_t* xh, const uint32_t* xl,
                                         const int32_t* bsum, uint32_t tlo, uint32_t thi, const uint2* grid_s) {
    if constexpr (FMT == IQK_IQ2_K) {
        const uint32_t q[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
        const uint32_t sc = r.a ^ 0x8888u;  // nibble ^ 8 read as signed 4-bit = nibble - 8
        const uint32_t sx = r.b >> (4 * (c & 1));
        // all four sub-blocks' weights first, then eight interleaved dot
        // chains (hi/lo x 4 sub-blocks), so dependent ops are not adjacent
        uint32_t w[4][4];
        uint32_t m[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) m[i] = (uint32_t)__builtin_amdgcn_sbfe((int)sx, i, 1) & 0x04040404u;
        expand_pair(q[0], q[1], m[0], m[1], tlo, thi, w[0], w[1]);
        expand_pair(q[2], q[3], m[2], m[3], tlo, thi, w[2], w[3]);
        int h[4], l[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            h[i] = dot4_first(w[i][0], xh[4 * i]);
            l[i] = dot4_first(w[i][0], xl[4 * i]);
        }
#pragma unroll
        for (int jj = 1; jj < 4; ++jj)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                h[i] = __builtin_amdgcn_sdot4((int)w[i][jj], (int)xh[4 * i + jj], h[i], false);
                l[i] = __builtin_amdgcn_sdot4((int)w[i][jj], (int)xl[4 * i + jj], l[i], false);
            }
        int ah = 0, al = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int si = __builtin_amdgcn_sbfe((int)sc, 4 * i, 4);
            ah += __mul24(h[i], si);
            al += __mul24(l[i], si);
        }
        return (float)(ah * 256 + al);  // exact: |.| < 2^31, one rounding as before
    } else if constexpr (FMT == IQK_IQ2_KS) {
        const uint32_t q[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
        const int sh = 2 * (c & 3);
        const uint32_t schx = ~r.b;  // high bit flipped: the 5-bit field read signed = raw - 16
        int ah = 0, al = 0;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const uint32_t raw = ((r.a >> (4 * s)) & 15u) | (((schx >> (sh + s)) & 1u) << 4);
            const int si = __builtin_amdgcn_sbfe((int)raw, 0, 5);
            const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)r.c, sh + s, 1) & 0x04040404u;
            uint32_t w0[4], w1[4];
            expand_pair(q[2 * s], q[2 * s + 1], m, m, tlo, thi, w0, w1);
            int h = dot16w<true>(w0, xh + 8 * s, 0);
            h = dot16w<false>(w1, xh + 8 * s + 4, h);
            int l = dot16w<true>(w0, xl + 8 * s, 0);
            l = dot16w<false>(w1, xl + 8 * s + 4, l);
            ah += __mul24(h, si);
            al += __mul24(l, si);
        }
        return (float)(ah * 256 + al);  // exact: |.| < 2^31, one rounding as before
    } else {
        float part = 0.f;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const uint32_t h16 = (r.a >> (16 * b)) & 0xFFFFu;
            const uint32_t qsw = b == 0 ? r.q.x : r.q.y;
            int ah = 0, al = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int g = 4 * b + j;
                const uint32_t idx = ((qsw >> (8 * j)) & 0xFFu) | (((h16 >> (3 * j)) & 7u) << 8);
                const uint2 gv = grid_s[idx];
                // (the chain's first dot starts from an inline zero: no v_mov)
                ah = j == 0 ? dot4_first(gv.x, xh[2 * g]) : __builtin_amdgcn_sdot4((int)gv.x, (int)xh[2 * g], ah, false);
                ah = __builtin_amdgcn_sdot4((int)gv.y, (int)xh[2 * g + 1], ah, false);
                al = j == 0 ? dot4_first(gv.x, xl[2 * g]) : __builtin_amdgcn_sdot4((int)gv.x, (int)xl[2 * g], al, false);
                al = __builtin_amdgcn_sdot4((int)gv.y, (int)xl[2 * g + 1], al, false);
            }
            const float shift = (h16 >> 15) ? -0.125f : 0.125f;
            const float tb = (float)(ah * 256 + al) + shift * (float)bsum[b];
            part += tb * (float)(2 * ((h16 >> 12) & 7u) + 1);
        }
        return part;
    }
}

template <int FMT, int N>
struct Group {
    RowData r[Geo<N>::GIT];
};

// Rows of one unit: local row q = it * RPI + lane_row maps to an expert row
// through `row_of` (identity plus offset, or the gate/up split).  A launch
// reads each row once, so the loads carry the non-temporal hint: measured on
// one-token launches, 10.5 -> 9.7 us (IQ2_K gate/up) and 7.0 -> 6.1 us
// (down), the floor variant likewise, while the small data every launch
// re-reads (activation, ids, grid) is no longer pushed out of the L2 by the
// streamed rows.  (The fused prefill, whose tiles share rows through the L2,
// is slower with it and keeps the default.)
template <int FMT, int N, class RowOf>
__device__ __forceinline__ void load_group(Group<FMT, N>& g, const ExpertRes& res, RowOf row_of, int lane_row, int c) {
    using G = Geo<N>;
    constexpr bool kScalarD = (FMT == IQK_IQ2_KS || FMT == IQK_IQ1_S_R4) && (G::LPR == 64 || G::LPR == 32);
#pragma unroll
    for (int it = 0; it < G::GIT; ++it) {
        g.r[it] = load_row<FMT, N, kNonTemporal, kScalarD>(res, (uint32_t)row_of(it * G::RPI + lane_row), (uint32_t)c);
        if constexpr (kScalarD) {
            // the per-row scale is the same for every lane of a row, so it is
            // one scalar load per row instead of a vector load per lane:
            // measured 9.7 -> 9.3 us (IQ2_KS gate/up, one token) and
            // 5.6 -> 5.4 us (IQ1_S_R4 down); rows past the last one clamp to
            // it (their sums are never stored)
            auto dof = [&](int qq) {
                const uint32_t r = (uint32_t)row_of(it * G::RPI + qq);
                return sload_u16(res.dp + 2u * (r < res.dmax ? r : res.dmax));
            };
            if constexpr (G::LPR == 64) g.r[it].d = dof(0);
            else {
                const uint32_t d0 = dof(0), d1 = dof(1);
                g.r[it].d = lane_row ? d1 : d0;
            }
        }
    }
}

// float -> bf16, round to nearest even (NaN stays a quiet NaN)
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Position of one item: its outer index (pair, or token for kCombine), its
// unit inside the outer, and the slot j (kCombine).  Items of a wave are
// visited in increasing order, nwaves apart, so the cursor advances without
// a division: units step through the outers (kPlain, kSwiGLU), slots step
// through the units of the block's one token (kCombine).
struct Cursor {
    int outer, rem, j;
    template <int MODE>
    __device__ __forceinline__ void advance(int step, int upo, int k) {
        if constexpr (MODE == kCombine) {
            j += step;
            while (j >= k) {
                j -= k;
                ++rem;
            }
        } else {
            rem += step;
            while (rem >= upo) {
                rem -= upo;
                ++outer;
            }
        }
    }
};

// kCombine: units per block at most, so the per-slot partial sums of a block
// fit in LDS (units * k * rows per unit floats)
constexpr int kCombineMaxUnits = 64;

// Pairs (and activation rows) one workgroup may span; the launch plan keeps
// every block within it.  Each spanned activation row has its own
// fixed-point copy in LDS.
template <int MODE>
constexpr int max_x_rows() { return MODE == kCombine ? 8 : 4; }

template <int FMT, int N, int XDT, bool FLOOR, int MODE>
__global__ __launch_bounds__(64 * kMaxWaves) void gemv_kernel(GemvParams p) {
    using G = Geo<N>;
    constexpr int kMaxX = max_x_rows<MODE>();
    __shared__ XLds<N> X[kMaxX];
    __shared__ uint2 grid_s[FMT == IQK_IQ1_S_R4 ? 2048 : 1];

    const int nthreads = blockDim.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nwaves = nthreads >> 6;
    const int bid = blockIdx.x;
    // Units are cut evenly over the blocks (kCombine: over the bpt blocks of
    // each token), so every CU gets the same number of rows.
    int u0, u1;
    if constexpr (MODE == kCombine) {
        const int t = (int)fdiv((uint32_t)bid, p.dbpt);
        const int lb = bid - t * p.bpt;
        u0 = t * p.upo + lb * p.ubase + min(lb, p.urem);
        u1 = u0 + p.ubase + (lb < p.urem ? 1 : 0);
    } else {
        u0 = bid * p.ubase + min(bid, p.urem);
        u1 = u0 + p.ubase + (bid < p.urem ? 1 : 0);
    }
    constexpr bool kSlots = MODE == kCombine;   // k items per unit
    const int kk = kSlots ? p.k : 1;
    const int o_first = (int)fdiv((uint32_t)u0, p.dupo);
    const int o_last = (int)fdiv((uint32_t)(u1 - 1), p.dupo);
    __shared__ float part_s[MODE == kCombine ? kCombineMaxUnits * 8 * 8 : 1];  // [unit][slot][row]
    auto pair_of = [&](int outer, int j) { return kSlots ? outer * p.k + j : outer; };
    // activation row of a pair: x[t] when shared by the k slots, else x[t, j]
    auto xrow_of = [&](int pair) { return p.x_slots == 1 ? (int)fdiv((uint32_t)pair, p.dk) : pair; };
    const int xr0 = xrow_of(pair_of(o_first, 0));
    const int nx = xrow_of(pair_of(o_last, kk - 1)) - xr0 + 1;
    // The ids (and router weights) of every pair the block touches, staged
    // in LDS at the start: read from memory later, after the first result
    // store, every read would be a vector load that waits for all the row
    // loads in flight.
    constexpr int kPairs = max_x_rows<MODE>();
    __shared__ int32_t ids_s[kPairs];
    __shared__ float rw_s[kPairs];
    const int pr0 = pair_of(o_first, 0);
    const int pr_last = pair_of(o_last, kk - 1);

    const int c = lane % G::LPR;  // chunk of k owned by this lane
    const int lane_row = lane / G::LPR;

    // The activation (and the IQ1_S_R4 grid) is on the critical path: every
    // first-pass load is issued before any of them is waited for.
    auto xrow_ptr = [&](int i) {
        const int64_t xoff = (int64_t)(xr0 + i / (N / 16)) * N;
        return XDT == IQK_BF16 ? (const void*)((const uint16_t*)p.x + xoff) : (const void*)((const float*)p.x + xoff);
    };
    const int xtotal = nx * (N / 16);
    XRaw<XDT> xraw;
    if (tid < xtotal) xraw = load_xblock<N, XDT>(xrow_ptr(tid), tid % (N / 16));
    uint4 gw0, gw1;
    const uint4* gsrc = (const uint4*)p.grid;
    uint4* gdst = (uint4*)grid_s;
    if constexpr (FMT == IQK_IQ1_S_R4) {
        if (tid < 1024) gw0 = gsrc[tid];
        if (tid + nthreads < 1024) gw1 = gsrc[tid + nthreads];
    }
    int32_t id_v = 0;
    float rw_v = 0.f;
    if (tid < kPairs) {
        id_v = p.ids[min(pr0 + tid, pr_last)];
        if constexpr (MODE == kCombine) rw_v = p.rw[min(pr0 + tid, pr_last)];
    }
    if (tid < xtotal) prep_block<FMT, N, XDT>(xraw, X[tid / (N / 16)], tid % (N / 16));
    if (tid < kPairs) {
        ids_s[tid] = id_v;
        rw_s[tid] = rw_v;
    }
    for (int i = tid + nthreads; i < xtotal; i += nthreads)
        prep_block<FMT, N, XDT>(load_xblock<N, XDT>(xrow_ptr(i), i % (N / 16)), X[i / (N / 16)], i % (N / 16));
    if constexpr (FMT == IQK_IQ1_S_R4) {
        if (tid < 1024) gdst[tid] = gw0;
        if (tid + nthreads < 1024) gdst[tid + nthreads] = gw1;
        for (int i = tid + 2 * nthreads; i < 1024; i += nthreads) gdst[i] = gsrc[i];
    }
    lds_barrier();

    const int nunits = u1 - u0;
    const int nitems = nunits * kk;
    const int my_items = wave < nitems ? (nitems - wave + nwaves - 1) / nwaves : 0;
    if constexpr (MODE != kCombine) {
        if (my_items == 0) return;
    }
    const int rem0 = u0 - o_first * p.upo;  // first unit of the block inside its outer
    Cursor lc;  // next item to load
    if constexpr (MODE == kCombine) {
        const int ul = (int)fdiv((uint32_t)wave, p.dk);
        lc.outer = o_first;
        lc.rem = rem0 + ul;
        lc.j = wave - ul * p.k;
    } else {
        lc.outer = (int)fdiv((uint32_t)(u0 + wave), p.dupo);
        lc.rem = u0 + wave - lc.outer * p.upo;
        lc.j = 0;
    }
    Cursor pc = lc;  // next item to process

    constexpr int kHalf = G::RPG / 2;
    const int half_out = p.out >> 1;
    // expert row of local row q of the unit `rem`
    auto unit_row = [&](int rem, int q) {
        if constexpr (MODE == kSwiGLU) return q < kHalf ? rem * kHalf + q : half_out + rem * kHalf + (q - kHalf);
        else return rem * G::RPG + q;
    };
    auto expert_of = [&](int pair) { return __builtin_amdgcn_readfirstlane(ids_s[pair - pr0]); };

    // Loads of an item past the wave's last use a zero-record resource.
    auto load_next = [&](Group<FMT, N>& buf, bool live) {
        const ExpertRes res = expert_res<FMT, N>(p, live ? expert_of(pair_of(lc.outer, lc.j)) : -1);
        const int rem = lc.rem;
        load_group<FMT, N>(buf, res, [&](int q) { return unit_row(rem, q); }, lane_row, c);
        lc.template advance<MODE>(nwaves, p.upo, p.k);
    };
    // The first two items' rows are requested only now: issued earlier, the
    // launch's row traffic would queue ahead of the activation reads and
    // hold every wave at the barrier until most rows had streamed in.
    Group<FMT, N> bufA, bufB;
    load_next(bufA, my_items > 0);
    load_next(bufB, my_items > 1);

    uint32_t xh[16], xl[16];
    float lane_scale = 0.f;
    int32_t bsum[2] = {0, 0};
    int cur_x = -1;
    auto load_x = [&](int xi) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 a = *(const uint4*)&X[xi].hi[4 * xslot(c, i)];
            const uint4 b = *(const uint4*)&X[xi].lo[4 * xslot(c, i)];
            xh[4 * i] = a.x; xh[4 * i + 1] = a.y; xh[4 * i + 2] = a.z; xh[4 * i + 3] = a.w;
            xl[4 * i] = b.x; xl[4 * i + 1] = b.y; xl[4 * i + 2] = b.z; xl[4 * i + 3] = b.w;
        }
        lane_scale = X[xi].scale[c] * p.tab_scale;
        if constexpr (FMT == IQK_IQ1_S_R4) {
            bsum[0] = X[xi].bsum[2 * c];
            bsum[1] = X[xi].bsum[2 * c + 1];
        }
        cur_x = xi;
    };

    auto process = [&](const Group<FMT, N>& gb) {
        const int outer = pc.outer;
        const int rem = pc.rem;
        const int j = pc.j;
        pc.template advance<MODE>(nwaves, p.upo, p.k);
        const int pair = pair_of(outer, j);
        const bool valid = (unsigned)expert_of(pair) < (unsigned)p.E;
        const int xi = xrow_of(pair) - xr0;
        if (xi != cur_x) load_x(xi);
        uint32_t part[G::GIT];
#pragma unroll
        for (int it = 0; it < G::GIT; ++it) {
            if constexpr (FLOOR) {
                part[it] = gb.r[it].q.x ^ gb.r[it].q.y ^ gb.r[it].q.z ^ gb.r[it].q.w ^ gb.r[it].a ^
                           (gb.r[it].b << 8) ^ (gb.r[it].c << 16) ^ (gb.r[it].d << 3) ^ xh[it & 15];
            } else {
                const float f = row_dot<FMT>(gb.r[it], c, xh, xl, bsum, p.tab_lo, p.tab_hi, grid_s);
                part[it] = __float_as_uint(f * (half_to_float(gb.r[it].d) * lane_scale));
            }
        }
        int q;
        bool writer;
        uint32_t sum = reduce_group<N, FLOOR>(part, lane, &q, &writer);
        // invalid id: its rows read zeros; they are reported as NaN (all ones
        // in the floor variant)
        if (!valid) sum = FLOOR ? 0xFFFFFFFFu : 0x7FC00000u;
        if constexpr (MODE == kPlain) {
            const int r = unit_row(rem, q);
            void* ybase = FLOOR ? (void*)(p.sink + (int64_t)pair * p.out) : (void*)(p.y + (int64_t)pair * p.out);
            const Rsrc yres = make_rsrc(ybase, (uint32_t)p.out * 4u);
            __builtin_amdgcn_raw_buffer_store_b32(sum, yres, writer ? (uint32_t)r * 4u : kOob, 0, 0);
        } else if constexpr (MODE == kSwiGLU) {
            // gate row q < RPG/2 and its up row q + RPG/2 sit 32 lanes apart
            // (16 when a row spans 32 lanes)
            // (a lane swap on the VALU: the second half of the pair holds, in
            // the gate row's lanes, the other row group's value)
            uint32_t up;
            if constexpr (G::LPR == 32) up = __builtin_amdgcn_permlane16_swap(sum, sum, false, false)[1];
            else up = __builtin_amdgcn_permlane32_swap(sum, sum, false, false)[1];
            const float g = __uint_as_float(sum);
            const float hv = silu_mul(g, __uint_as_float(up));
            const int r = rem * kHalf + q;  // h index inside the pair
            const Rsrc hres = make_rsrc(p.h + (int64_t)pair * half_out, (uint32_t)half_out * 2u);
            __builtin_amdgcn_raw_buffer_store_b16((unsigned short)f32_to_bf16(hv), hres,
                                                  writer && q < kHalf ? (uint32_t)r * 2u : kOob, 0, 0);
        } else {
            // slot partial, weighted; summed over the slots in order below
            const float w = rw_s[pair - pr0];
            if (writer) part_s[((rem - rem0) * p.k + j) * G::RPG + q] = w * __uint_as_float(sum);
        }
    };

    // Items 0 and 1 are in flight.  The loop refills a buffer just before
    // processing the other one, so at its top exactly one item's loads are
    // outstanding on every path and each wait covers only the item it needs.
    if (MODE != kCombine || my_items > 0) {  // other modes returned above when idle
        load_x(xrow_of(pair_of(pc.outer, pc.j)) - xr0);
        process(bufA);
        bool loop = true;
        if constexpr (FMT == IQK_IQ1_S_R4) {
            // measured: at one or two items per wave the IQ1_S_R4 instance is
            // faster without the loop's dead refills (the 2-bit ones are not)
            if (my_items <= 2) {
                if (my_items == 2) process(bufB);
                loop = false;
            }
        }
        for (int i = 1; loop && i < my_items; i += 2) {
            load_next(bufA, i + 1 < my_items);
            process(bufB);
            load_next(bufB, i + 2 < my_items);
            if (i + 1 >= my_items) break;
            process(bufA);
        }
    }

    if constexpr (MODE == kCombine) {
        // y[t, row] = sum over slots in order j = 0..k-1 of the weighted partials
        lds_barrier();
        for (int i = tid; i < nunits * G::RPG; i += nthreads) {
            const int ul = i / G::RPG;
            const int q = i - ul * G::RPG;
            const int row = (rem0 + ul) * G::RPG + q;
            if (row < p.out) {
                float acc = part_s[(ul * p.k) * G::RPG + q];
                for (int j = 1; j < p.k; ++j) acc += part_s[(ul * p.k + j) * G::RPG + q];
                p.y[(int64_t)o_first * p.out + row] = acc;
            }
        }
    }
}

template <int FMT, int N, int XDT, bool FLOOR, int MODE>
hipError_t launch_inst(GemvParams p, int64_t T, hipStream_t s) {
    using G = Geo<N>;
    // units: rows of one outer in reduction groups (kSwiGLU: RPG/2 output rows)
    const int64_t out_rows = MODE == kSwiGLU ? p.out / 2 : p.out;
    const int64_t rows_per_unit = MODE == kSwiGLU ? G::RPG / 2 : G::RPG;
    const int64_t upo = (out_rows + rows_per_unit - 1) / rows_per_unit;
    const int64_t outers = MODE == kCombine ? T : T * p.k;
    const int64_t total = outers * upo;
    if (total <= 0 || total > 0x7FFFFFFF) return hipErrorInvalidValue;
    int64_t nb, bpt = 1;
    if constexpr (MODE == kCombine) {
        // blocks never straddle tokens (a block holds one token's k
        // activation rows) and hold at most kCombineMaxUnits units
        bpt = IQK_GEMV_TARGET_BLOCKS / T;
        const int64_t bpt_lds = (upo + kCombineMaxUnits - 1) / kCombineMaxUnits;
        bpt = bpt < bpt_lds ? bpt_lds : bpt;
        bpt = bpt < 1 ? 1 : (bpt > upo ? upo : bpt);
        nb = T * bpt;
        p.ubase = (int32_t)(upo / bpt);
        p.urem = (int32_t)(upo % bpt);
    } else {
        // one large workgroup per CU over the whole call -- or two smaller
        // ones when each then holds at most 16 groups (at most 8 waves, so
        // both stay resident on the CU): measured faster for a one-token
        // launch, where two blocks' start-ups overlap the other's decode;
        // more blocks only when a block would otherwise span more than
        // max_x_rows pairs
        int64_t target = IQK_GEMV_TARGET_BLOCKS;
        if (total <= 2 * target * 16) target *= 2;
        nb = total < target ? total : target;
        // a block of at most (span - 1) * upo + 1 units touches at most span outers
        const int64_t span_units = (max_x_rows<MODE>() - 1) * upo + 1;
        const int64_t nb_span = (total + span_units - 1) / span_units;
        nb = nb < nb_span ? nb_span : nb;
        p.ubase = (int32_t)(total / nb);
        p.urem = (int32_t)(total % nb);
    }
    const int64_t units = MODE == kCombine ? (upo + bpt - 1) / bpt : (total + nb - 1) / nb;  // largest block
    const int64_t items = MODE == kCombine ? units * p.k : units;
    // waves: a multiple of four (one share per SIMD) up to 16, at least
    // IQK_GEMV_MIN_GROUPS items each once the block is large enough (kCombine:
    // one item each, up to 16 -- its block is the CU's only one, and must
    // convert all k activation rows first; measured 8.5 -> 8.1 us for a
    // one-token down projection)
    int64_t waves = MODE == kCombine ? items : (items + IQK_GEMV_MIN_GROUPS - 1) / IQK_GEMV_MIN_GROUPS;
    waves = items < 4 ? items : ((waves + 3) / 4) * 4;
    waves = waves > kMaxWaves ? kMaxWaves : (waves < 1 ? 1 : waves);
    p.outers = (int32_t)outers;
    p.upo = (int32_t)upo;
    p.bpt = (int32_t)bpt;
    p.dupo = make_fastdiv((uint32_t)upo);
    p.dk = make_fastdiv((uint32_t)p.k);
    p.dbpt = make_fastdiv((uint32_t)bpt);
    hipLaunchKernelGGL((gemv_kernel<FMT, N, XDT, FLOOR, MODE>), dim3((unsigned)nb), dim3((unsigned)(64 * waves)), 0, s, p);
    return hipGetLastError();
}

template <int FMT, int N, bool FLOOR, int MODE>
hipError_t launch_x(const GemvParams& p, int xdt, int64_t T, hipStream_t s) {
    if (xdt == IQK_BF16) return launch_inst<FMT, N, IQK_BF16, FLOOR, MODE>(p, T, s);
    return launch_inst<FMT, N, IQK_F32, FLOOR, MODE>(p, T, s);
}

template <int FMT, bool FLOOR, int MODE>
hipError_t launch_n(const GemvParams& p, int64_t n, int xdt, int64_t T, hipStream_t s) {
    if (n == 4096) return launch_x<FMT, 4096, FLOOR, MODE>(p, xdt, T, s);
    if (n == 2048) return launch_x<FMT, 2048, FLOOR, MODE>(p, xdt, T, s);
    return launch_x<FMT, 512, FLOOR, MODE>(p, xdt, T, s);
}

template <bool FLOOR, int MODE>
hipError_t launch_fmt(const GemvParams& p, int fmt, int64_t n, int xdt, int64_t T, hipStream_t s) {
    if (fmt == IQK_IQ2_KS) return launch_n<IQK_IQ2_KS, FLOOR, MODE>(p, n, xdt, T, s);
    if (fmt == IQK_IQ2_K) return launch_n<IQK_IQ2_K, FLOOR, MODE>(p, n, xdt, T, s);
    return launch_n<IQK_IQ1_S_R4, FLOOR, MODE>(p, n, xdt, T, s);
}

// ---------------------------------------------------------------------------
// Grouped decode matvec: the pairs routed to one expert in one pass over its
// rows.  Each 64-weight chunk is decoded once into int8 weight words and
// then multiplied with every token of the pass, so the decode (and the HBM
// read) is shared by the expert's tokens.  A lane's chunk of k is the same
// for every row it visits, so the pass's activations live in its registers
// (converted by the lane itself) and the inner loop touches no LDS.
// ---------------------------------------------------------------------------

constexpr int kGWaves = 8;  // waves per workgroup (256 registers per lane)
// tokens per pass over an expert's rows: their activations stay in
// registers (a float32 activation needs more registers to convert)
template <int XDT>
constexpr int grouped_tok() { return XDT == IQK_BF16 ? 4 : 3; }

struct GroupedParams {
    const uint8_t* S;
    int64_t off0, off1, off2, off3, off4;
    int32_t E, out;
    uint32_t tab_lo, tab_hi;
    float tab_scale;
    const int8_t* grid;
    const void* x;
    int32_t x_slots, k;
    const int32_t* offsets;  // [E + 1] from the routing gather
    const int32_t* perm;     // expert-sorted pair indices
    const int64_t* plan;     // [E + 1] cost prefix
    float* y;                // [T * k, out]
    int64_t y_bytes;
    int32_t upo;             // reduction groups per expert
};

// One lane's 64 activations of one token, in the fixed point of the per-pair
// matvec (the same scale, bytes and word order as its LDS copy).
struct XLane {
    uint32_t hi[16], lo[16];
    float scale;       // 2^(emax - 13) times the table scale
    int32_t bsum[2];   // IQ1_S_R4: sums of the fixed-point values per 32
};

template <int XDT>
__device__ __forceinline__ void lane_block(const void* xrow, int c, int blk, float* v) {
    if constexpr (XDT == IQK_BF16) {
        const uint4* src = (const uint4*)xrow + 8 * c + 2 * blk;
        const uint4 a = src[0], b = src[1];
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
        const uint4* src = (const uint4*)xrow + 16 * c + 4 * blk;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 a = src[i];
            v[4 * i] = __uint_as_float(a.x);
            v[4 * i + 1] = __uint_as_float(a.y);
            v[4 * i + 2] = __uint_as_float(a.z);
            v[4 * i + 3] = __uint_as_float(a.w);
        }
    }
}

// (two passes over the 64 values, 16 at a time: the maximum, then the
// conversion; the second pass reads them again from the cache)
template <int FMT, int XDT>
__device__ __forceinline__ void lane_x(const void* xrow, int c, float tab_scale, XLane& o) {
    float am = 0.f;
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
        float v[16];
        lane_block<XDT>(xrow, c, blk, v);
#pragma unroll
        for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(v[i]));
    }
    const uint32_t amax = __float_as_uint(am);
    int emax = (int)(amax >> 23) - 127;
    emax = emax < -100 ? -100 : emax;
    const float sc = __builtin_ldexpf(1.0f, 13 - emax);
    // the per-pair matvec's conversion (prep_block): q = rint(v sc) through
    // one fma against 1.5 2^23, planes as byte gathers of q
    uint32_t bs[2] = {0u - 32u * 0x4B400000u, 0u - 32u * 0x4B400000u};
#pragma unroll
    for (int blk = 0; blk < 4; ++blk) {
        float v[16];
        lane_block<XDT>(xrow, c, blk, v);
        uint32_t q[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            q[i] = __float_as_uint(__builtin_fmaf(v[i], sc, 12582912.0f));  // 0x4B400000 + q, |q| <= 2^14
            bs[blk >> 1] += q[i];
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int i0 = FMT == IQK_IQ1_S_R4 ? 4 * j : j;
            const int st = FMT == IQK_IQ1_S_R4 ? 1 : 4;
            const uint32_t w01 = __builtin_amdgcn_perm(q[i0 + st], q[i0], 0x05040100u);
            const uint32_t w23 = __builtin_amdgcn_perm(q[i0 + 3 * st], q[i0 + 2 * st], 0x05040100u);
            o.lo[4 * blk + j] = __builtin_amdgcn_perm(w23, w01, 0x06040200u);
            o.hi[4 * blk + j] =
                __builtin_amdgcn_perm(add_u16x2(w23, 0x00800080u), add_u16x2(w01, 0x00800080u), 0x07050301u);
        }
    }
    o.scale = __builtin_ldexpf(1.0f, emax - 13) * tab_scale;
    o.bsum[0] = (int32_t)bs[0];
    o.bsum[1] = (int32_t)bs[1];
}

// One lane's decoded 64-weight chunk of one row: int8 weight words w[i]
// (word i pairs with activation word i of the chunk), the sub-block scale
// indices (2-bit members), the block scales and shifts (IQ1_S_R4), the row
// scale.
struct Dec {
    uint32_t w[16];
    int si[4];
    float fs[2], fh[2];
    float d;
};

template <int FMT>
__device__ __forceinline__ void decode_chunk(Dec& o, const RowData& r, int c, uint32_t tlo, uint32_t thi,
                                             const uint2* grid_s) {
    o.d = half_to_float(r.d);
    if constexpr (FMT == IQK_IQ2_K) {
        const uint32_t q[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
        const uint32_t sc = r.a ^ 0x8888u;
        const uint32_t sx = r.b >> (4 * (c & 1));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)sx, i, 1) & 0x04040404u;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                o.w[4 * i + jj] = __builtin_amdgcn_perm(thi, tlo, and_or_fast(q[i] >> (2 * jj), 0x03030303u, m));
            o.si[i] = __builtin_amdgcn_sbfe((int)sc, 4 * i, 4);
        }
    } else if constexpr (FMT == IQK_IQ2_KS) {
        const uint32_t q[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
        const int sh = 2 * (c & 3);
        const uint32_t schx = ~r.b;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const uint32_t raw = ((r.a >> (4 * s)) & 15u) | (((schx >> (sh + s)) & 1u) << 4);
            o.si[s] = __builtin_amdgcn_sbfe((int)raw, 0, 5);
            const uint32_t m = (uint32_t)__builtin_amdgcn_sbfe((int)r.c, sh + s, 1) & 0x04040404u;
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    o.w[4 * (2 * s + t) + jj] =
                        __builtin_amdgcn_perm(thi, tlo, and_or_fast(q[2 * s + t] >> (2 * jj), 0x03030303u, m));
        }
    } else {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const uint32_t h16 = (r.a >> (16 * b)) & 0xFFFFu;
            const uint32_t qsw = b == 0 ? r.q.x : r.q.y;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int g = 4 * b + j;
                const uint32_t idx = ((qsw >> (8 * j)) & 0xFFu) | (((h16 >> (3 * j)) & 7u) << 8);
                const uint2 gv = grid_s[idx];
                o.w[2 * g] = gv.x;
                o.w[2 * g + 1] = gv.y;
            }
            o.fh[b] = (h16 >> 15) ? -0.125f : 0.125f;
            o.fs[b] = (float)(2 * ((h16 >> 12) & 7u) + 1);
        }
    }
}

// The decoded chunk against one token's activations, before the per-lane
// float scale: the same integer sums and float steps as the per-pair matvec.
template <int FMT>
__device__ __forceinline__ float dot_chunk(const Dec& o, const XLane& x) {
    int h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h[i] = dot4_first(o.w[4 * i], x.hi[4 * i]);
        l[i] = dot4_first(o.w[4 * i], x.lo[4 * i]);
#pragma unroll
        for (int jj = 1; jj < 4; ++jj) {
            h[i] = __builtin_amdgcn_sdot4((int)o.w[4 * i + jj], (int)x.hi[4 * i + jj], h[i], false);
            l[i] = __builtin_amdgcn_sdot4((int)o.w[4 * i + jj], (int)x.lo[4 * i + jj], l[i], false);
        }
    }
    if constexpr (FMT == IQK_IQ2_K) {
        int ah = 0, al = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ah += __mul24(h[i], o.si[i]);
            al += __mul24(l[i], o.si[i]);
        }
        return (float)ah * 256.0f + (float)al;
    } else if constexpr (FMT == IQK_IQ2_KS) {
        int ah = 0, al = 0;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            ah += __mul24(h[2 * s] + h[2 * s + 1], o.si[s]);
            al += __mul24(l[2 * s] + l[2 * s + 1], o.si[s]);
        }
        return (float)ah * 256.0f + (float)al;
    } else {
        float part = 0.f;
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const int ah = h[2 * b] + h[2 * b + 1], al = l[2 * b] + l[2 * b + 1];
            const float tb = (float)ah * 256.0f + (float)al + o.fh[b] * (float)x.bsum[b];
            part += tb * o.fs[b];
        }
        return part;
    }
}

// Cost of one reduction group of an expert with M tokens: a decode per pass
// of up to MT tokens plus one multiply per token (decode about 5/3 of a
// token's multiply in instructions).
template <int MT>
__device__ __forceinline__ int64_t grouped_unit_cost(int M) {
    return (int64_t)5 * ((M + MT - 1) / MT) + 3 * (int64_t)M;
}

// plan[e] = cost of all reduction groups of experts before e (one workgroup).
template <int MT>
__global__ __launch_bounds__(1024) void grouped_plan_kernel(const int32_t* offsets, int E, int upo, int64_t* plan) {
    __shared__ int64_t part[1024];
    const int tid = threadIdx.x;
    int64_t carry = 0;
    if (tid == 0) plan[0] = 0;
    for (int c0 = 0; c0 < E; c0 += 1024) {
        const int e = c0 + tid;
        part[tid] = e < E ? grouped_unit_cost<MT>(offsets[e + 1] - offsets[e]) * upo : 0;
        __syncthreads();
        for (int o = 1; o < 1024; o <<= 1) {
            const int64_t add = tid >= o ? part[tid - o] : 0;
            __syncthreads();
            part[tid] += add;
            __syncthreads();
        }
        if (e < E) plan[e + 1] = carry + part[tid];
        carry += part[1023];
        __syncthreads();
    }
}

// Workgroup b of G takes the reduction groups whose cost range starts in
// [b C / G, (b + 1) C / G), C = plan[E]: a contiguous run over the
// expert-sorted list, so a workgroup converts each expert's activations
// once per pass and spans few experts.
template <int FMT, int N, int XDT>
__global__ __launch_bounds__(64 * kGWaves) void gemv_grouped_kernel(GroupedParams p) {
    using G = Geo<N>;
    constexpr int kGTok = grouped_tok<XDT>();
    __shared__ uint2 grid_s[FMT == IQK_IQ1_S_R4 ? 2048 : 1];
    __shared__ int32_t e_first;
    __shared__ uint64_t cand;  // experts e0 .. e0 + 63 with groups in this block
    __shared__ int32_t cand_g[64][2];
    __shared__ int32_t more;

    const int nthreads = blockDim.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nwaves = nthreads >> 6;
    const int64_t C = p.plan[p.E];
    const int64_t lo = C * blockIdx.x / gridDim.x, hi = C * (blockIdx.x + 1) / gridDim.x;
    if (lo >= hi) return;

    if constexpr (FMT == IQK_IQ1_S_R4) {
        for (int i = tid; i < 1024; i += nthreads) ((uint4*)grid_s)[i] = ((const uint4*)p.grid)[i];
    }
    for (int e = tid; e < p.E; e += nthreads)
        if (p.plan[e] <= lo && p.plan[e + 1] > lo) e_first = e;
    __syncthreads();

    const int c = lane % G::LPR;  // chunk of k owned by this lane
    const int lane_row = lane / G::LPR;
    const Rsrc yres = make_rsrc(p.y, (uint32_t)p.y_bytes);
    auto xrow_ptr = [&](int xr) {
        const int64_t xoff = (int64_t)xr * N;
        return XDT == IQK_BF16 ? (const void*)((const uint16_t*)p.x + xoff) : (const void*)((const float*)p.x + xoff);
    };

    for (int e0 = e_first;; e0 += 64) {
        if (wave == 0) {
            const int e = e0 + lane;
            int g0 = 0, g1 = 0;
            if (e < p.E) {
                const int64_t a = p.plan[e];
                const int64_t cr = grouped_unit_cost<kGTok>(p.offsets[e + 1] - p.offsets[e]);
                if (p.offsets[e + 1] > p.offsets[e] && a < hi) {
                    const int64_t s0 = lo > a ? (lo - a + cr - 1) / cr : 0;
                    const int64_t s1 = (hi - a + cr - 1) / cr;
                    g0 = (int)s0;
                    g1 = (int)(s1 < p.upo ? s1 : p.upo);
                }
            }
            cand_g[lane][0] = g0;
            cand_g[lane][1] = g1;
            const uint64_t m = __ballot(g0 < g1);
            if (lane == 0) {
                cand = m;
                more = e0 + 64 < p.E && p.plan[e0 + 64] < hi;
            }
        }
        __syncthreads();
        uint64_t cm = cand;
        const int go_on = more;
        while (cm) {
            const int j = __builtin_ctzll(cm);
            cm &= cm - 1;
            const int e = e0 + j;
            const int g0 = cand_g[j][0], g1 = cand_g[j][1];
            const int base = p.offsets[e];
            const int M = p.offsets[e + 1] - base;
            const ExpertRes res = expert_res<FMT, N>(p, e);
            const int ng = g1 - g0;
            const int my = wave < ng ? (ng - wave + nwaves - 1) / nwaves : 0;
            if (my == 0) continue;
            for (int ps = 0; ps < M; ps += kGTok) {
                const int mp = min(kGTok, M - ps);
                // rows of a group past `out` (and of a finished wave) read row
                // `out`, an out-of-range offset: zeros, never stored
                auto row_of = [&](int g, int it) { return g * G::RPG + it * G::RPI + lane_row; };
                Group<FMT, N> raw;
#pragma unroll
                for (int it = 0; it < G::GIT; ++it) {
                    const int r = row_of(g0 + wave, it);
                    raw.r[it] = load_row<FMT, N>(res, (uint32_t)(r < p.out ? r : p.out), (uint32_t)c);
                }
                // the pass's activations, this lane's chunk of each
                XLane xs[kGTok];
                int pr[kGTok];
#pragma unroll
                for (int mm = 0; mm < kGTok; ++mm) {
                    pr[mm] = 0;
                    if (mm < mp) {
                        const int pair = p.perm[base + ps + mm];
                        pr[mm] = pair;
                        lane_x<FMT, XDT>(xrow_ptr(p.x_slots == 1 ? pair / p.k : pair), c, p.tab_scale, xs[mm]);
                    }
                }
                for (int item = 0; item < my; ++item) {
                    const int g = g0 + wave + item * nwaves;
                    const int gn = g + nwaves;
                    const bool nlive = item + 1 < my;
                    float part[kGTok][G::GIT];
#pragma unroll
                    for (int it = 0; it < G::GIT; ++it) {
                        Dec dec;
                        decode_chunk<FMT>(dec, raw.r[it], c, p.tab_lo, p.tab_hi, grid_s);
                        // this row's slot now loads the same row of the next group
                        const int rn = row_of(gn, it);
                        raw.r[it] = load_row<FMT, N>(res, (uint32_t)(nlive && rn < p.out ? rn : p.out), (uint32_t)c);
#pragma unroll
                        for (int mm = 0; mm < kGTok; ++mm)
                            if (mm < mp) part[mm][it] = dot_chunk<FMT>(dec, xs[mm]) * (dec.d * xs[mm].scale);
                    }
#pragma unroll
                    for (int mm = 0; mm < kGTok; ++mm) {
                        if (mm < mp) {
                            uint32_t pu[G::GIT];
#pragma unroll
                            for (int it = 0; it < G::GIT; ++it) pu[it] = __float_as_uint(part[mm][it]);
                            int q;
                            bool writer;
                            const uint32_t sum = reduce_group<N, false>(pu, lane, &q, &writer);
                            const int row = g * G::RPG + q;
                            const uint32_t off = (uint32_t)(pr[mm] * p.out + row) * 4u;
                            __builtin_amdgcn_raw_buffer_store_b32(sum, yres, writer && row < p.out ? off : kOob, 0, 0);
                        }
                    }
                }
            }
        }
        if (!go_on) break;
        __syncthreads();  // every wave has read cand before wave 0 rewrites it
    }
}

int grouped_grid_blocks() {
    // one large workgroup per compute unit
    static int cu[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cu[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cu[dev] = n;
    }
    return cu[dev];
}

template <int FMT, int N, int XDT>
hipError_t launch_grouped_inst(GroupedParams p, hipStream_t s) {
    using G = Geo<N>;
    p.upo = (int32_t)((p.out + G::RPG - 1) / G::RPG);
    int64_t* plan = const_cast<int64_t*>(p.plan);
    hipLaunchKernelGGL((grouped_plan_kernel<grouped_tok<XDT>()>), dim3(1), dim3(1024), 0, s, p.offsets, (int)p.E,
                       (int)p.upo, plan);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((gemv_grouped_kernel<FMT, N, XDT>), dim3((unsigned)grouped_grid_blocks()), dim3(64 * kGWaves),
                       0, s, p);
    return hipGetLastError();
}

template <int FMT, int N>
hipError_t launch_grouped_x(const GroupedParams& p, int xdt, hipStream_t s) {
    if (xdt == IQK_BF16) return launch_grouped_inst<FMT, N, IQK_BF16>(p, s);
    return launch_grouped_inst<FMT, N, IQK_F32>(p, s);
}

template <int FMT>
hipError_t launch_grouped_n(const GroupedParams& p, int64_t n, int xdt, hipStream_t s) {
    if (n == 4096) return launch_grouped_x<FMT, 4096>(p, xdt, s);
    if (n == 2048) return launch_grouped_x<FMT, 2048>(p, xdt, s);
    return launch_grouped_x<FMT, 512>(p, xdt, s);
}

}  // namespace

hipError_t launch_gemv(const GemvLaunch& a, bool floor_variant, hipStream_t s) {
    GemvParams p;
    p.S = a.streams;
    p.off0 = a.pl.off[0];
    p.off1 = a.pl.off[1];
    p.off2 = a.pl.off[2];
    p.off3 = a.pl.off[3];
    p.off4 = a.pl.off[4];
    p.E = (int32_t)a.E;
    p.out = (int32_t)a.out;
    p.tab_lo = a.tab_lo;
    p.tab_hi = a.tab_hi;
    p.tab_scale = a.tab_scale;
    p.grid = a.grid;
    p.x = a.x;
    p.x_slots = a.x_slots;
    p.k = a.k;
    p.ids = a.ids;
    p.y = a.y;
    p.sink = a.sink;
    p.h = a.h;
    p.rw = a.route_w;
    p.outers = p.upo = p.ubase = p.urem = p.bpt = 0;
    if (floor_variant) return launch_fmt<true, kPlain>(p, a.fmt, a.n, a.x_dtype, a.T, s);
    if (a.mode == kSwiGLU) return launch_fmt<false, kSwiGLU>(p, a.fmt, a.n, a.x_dtype, a.T, s);
    if (a.mode == kCombine) return launch_fmt<false, kCombine>(p, a.fmt, a.n, a.x_dtype, a.T, s);
    return launch_fmt<false, kPlain>(p, a.fmt, a.n, a.x_dtype, a.T, s);
}

}  // namespace iqk

namespace iqk {

hipError_t launch_gemv_grouped(const GemvLaunch& a, const int32_t* offsets, const int32_t* perm, int64_t* plan,
                               hipStream_t s) {
    GroupedParams p;
    p.S = a.streams;
    p.off0 = a.pl.off[0];
    p.off1 = a.pl.off[1];
    p.off2 = a.pl.off[2];
    p.off3 = a.pl.off[3];
    p.off4 = a.pl.off[4];
    p.E = (int32_t)a.E;
    p.out = (int32_t)a.out;
    p.tab_lo = a.tab_lo;
    p.tab_hi = a.tab_hi;
    p.tab_scale = a.tab_scale;
    p.grid = a.grid;
    p.x = a.x;
    p.x_slots = a.x_slots;
    p.k = a.k;
    p.offsets = offsets;
    p.perm = perm;
    p.plan = plan;
    p.y = a.y;
    p.y_bytes = a.T * a.k * a.out * 4;
    p.upo = 0;
    if (a.fmt == IQK_IQ2_KS) return launch_grouped_n<IQK_IQ2_KS>(p, a.n, a.x_dtype, s);
    if (a.fmt == IQK_IQ2_K) return launch_grouped_n<IQK_IQ2_K>(p, a.n, a.x_dtype, s);
    return launch_grouped_n<IQK_IQ1_S_R4>(p, a.n, a.x_dtype, s);
}

}  // namespace iqk
