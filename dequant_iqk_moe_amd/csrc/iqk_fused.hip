// iqk_fused.hip -- prefill with the dequantization fused into the MFMA
// grouped GEMM.
//
// "mlx-iqk" package description, "Surface": a call with many token-expert
// pairs dequantizes the stacked experts to a dense type and multiplies with
// a grouped GEMM.  This path computes the same product without the dense
// copy: the bf16 weights are rebuilt from the compressed streams straight
// into MFMA operand registers, so each expert's compressed rows are read
// once and the 2-byte-per-weight round trip through HBM disappears.  The
// weights are the ones iqk_dequant writes ("Format": d * float(scale) *
// table value, or d * float(2 ls + 1) * (grid value + shift), float32, the
// two multiplications in that order, each rounded, then one
// round-to-nearest-even cast to bf16).  The IQ1_S_R4 grid must be ternary,
// as the grid is defined: a block's weights are looked up among the three
// values it can take; a grid holding any other value makes the output NaN.
//
// gfx950 design.
//   * A workgroup owns one expert and 256 weight rows; each of its 16 waves
//     owns a 16-row tile and walks k in steps of 256: lane (row r, group g)
//     reads the 64-weight chunk g of row r (the decode matvec's per-lane
//     loads) and turns it into eight 8-element B fragments of
//     v_mfma_f32_16x16x32_bf16.
//   * Per sub-block (16 weights for IQ2_K, 32 for IQ2_KS, 32 for IQ1_S_R4)
//     the lane builds a 4-entry bf16 table of its possible weights
//     (scale * table value, or scale * (grid value + shift)); each bf16 pair
//     of a fragment is then one v_perm_b32 of that table (two packed bf16
//     pairs), its selector one v_perm_b32 of doubled code bytes 2c and
//     2c + 1 (2-bit members: shifted and masked out of the code words;
//     IQ1_S_R4: its grid staged in LDS as doubled codes).  About 2-3 VALU
//     instructions per weight, once per weight whatever the number of
//     tokens.
//   * The expert's token rows (gathered through the routing permutation)
//     are staged in LDS (all of k for up to 16 tokens, 2048 k at a time for
//     up to 32), already in
//     the k order the fragments use (a per-step permutation that makes both
//     the table lookups and the LDS reads 16-byte contiguous); rows are
//     padded by 32 bytes against bank conflicts.  Each lane keeps the raw
//     words of the next four k steps in flight.
//   * Results go straight to y[t, j, :] (no scatter pass).
#include "iqk_device.h"

namespace iqk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#ifndef IQK_FUSED_WAVES
#define IQK_FUSED_WAVES 16
#endif
constexpr int kFWaves = IQK_FUSED_WAVES;    // waves per block, one 16-row tile each
constexpr int kFThreads = 64 * kFWaves;
constexpr int kFRows = 16 * kFWaves;        // weight rows per block
constexpr int kFMT = 2;                     // 16-token tiles per pass over k
constexpr int kFPad = 32;                   // LDS row padding (bank-conflict-free fragment reads)
// LDS for the staged token rows: one tile over all k up to 4096, or two
// tiles over 2048 k at a time
#ifndef IQK_FUSED_KC1
#define IQK_FUSED_KC1 4096  // k staged at a time for one token tile
#endif
constexpr int kFKC1 = IQK_FUSED_KC1;
constexpr int kFStageBytes = 32 * (2 * 2048 + kFPad) > 16 * (2 * kFKC1 + kFPad) ? 32 * (2 * 2048 + kFPad)
                                                                                : 16 * (2 * kFKC1 + kFPad);

struct FusedParams {
    const uint8_t* S;
    int64_t off0, off1, off2, off3, off4;
    int32_t E, out;
    float tab[8];            // value table (2-bit members)
    const int8_t* grid;      // IQ1_S_R4 grid [2048][8]
    const uint16_t* x;       // bf16 [T, x_slots, n]
    int32_t x_slots, k;
    const int32_t* offsets;  // [E + 1]
    const int32_t* perm;     // expert-sorted pair indices
    float* y;                // [T * k, out]
    int64_t y_bytes;
    const int64_t* plan;     // [E + 1] cost prefix (work plan)
};

// Workgroup barrier for LDS only: global loads issued before it stay in
// flight (a full __syncthreads would wait for them).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    const bf16x2 v = __builtin_convertvector(f32x2{a, b}, bf16x2);
    return __builtin_bit_cast(uint32_t, v);
}

// Selector picking bytes x and y of a word v and of a second word (bytes
// 4 + i of the perm source): [x, 4 + x, y, 4 + y].
constexpr uint32_t sel_pair(int x, int y) {
    return (uint32_t)x | (uint32_t)(4 + x) << 8 | (uint32_t)y << 16 | (uint32_t)(4 + y) << 24;
}

// A 4-entry bf16 table kept as two packed pairs (value c at bytes 2c and
// 2c + 1 of the 8 bytes {p23, p01}): a pair of weights with codes (a, b) is
// perm(p23, p01, [2a, 2a + 1, 2b, 2b + 1]), its selector one perm of the
// doubled codes v2 and v2 + 1 -- no byte split of the table is needed.
struct PairTab {
    uint32_t p01, p23;
};
__device__ __forceinline__ PairTab make_pair_tab(float v0, float v1, float v2, float v3) {
    return PairTab{pk_bf16(v0, v1), pk_bf16(v2, v3)};
}
__device__ __forceinline__ uint32_t pair_lookup(const PairTab& t, uint32_t v2, uint32_t v2p, uint32_t sel) {
    return __builtin_amdgcn_perm(t.p23, t.p01, __builtin_amdgcn_perm(v2p, v2, sel));
}

// The value table in vector registers, as named members: an array here
// would be turned into a private-memory lookup by the alphabet select.
struct Table8 {
    float v0, v1, v2, v3, v4, v5, v6, v7;
};

// The eight B fragments (4 dwords each) of one lane's 64-weight chunk, each
// handed to emit(fragment index, fragment) as soon as it is built.
// 2-bit members: fragment 2i + h holds weights (4h + d, 4h + d + 8) of code
// word i as dword d; IQ1_S_R4: fragment 2b + j holds group j of block b in
// natural order.
// PAIR_SHIFT (2-bit members): the codes of two words shifted together by one
// 64-bit shift per step (the bits crossing from the high word into the low
// one land outside every byte's 0x06 mask); measured at 512 tokens: IQ2_K
// down 245 -> 233 us, IQ2_KS gate/up 461 -> 447 us and down 237 -> 230 us,
// IQ2_K gate/up 0.6 % slower (it keeps one shift per word).
template <int FMT, bool PAIR_SHIFT, class Emit>
__device__ __forceinline__ void decode_chunk(const RowData& r, int c, const Table8& tv, const uint2* grid_s,
                                             Emit emit) {
    const float d = half_to_float(r.d);
    if constexpr (FMT == IQK_IQ2_K || FMT == IQK_IQ2_KS) {
        const uint32_t q[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
        auto table_of = [&](int i) {
            int si;
            bool alpha;
            if constexpr (FMT == IQK_IQ2_K) {
                si = __builtin_amdgcn_sbfe((int)(r.a ^ 0x8888u), 4 * i, 4);  // nibble - 8
                alpha = (r.b >> (4 * (c & 1) + i)) & 1u;
            } else {
                const int j = i >> 1;  // 32-weight sub-block
                const int sh = 2 * (c & 3) + j;
                si = (int)(((r.a >> (4 * j)) & 15u) | (((r.b >> sh) & 1u) << 4)) - 16;
                alpha = (r.c >> sh) & 1u;
            }
            const float s = d * (float)si;
            // alphabet select as one v_bfi_b32 per value (written as C the
            // compiler makes it two instructions, or a private-memory lookup)
            const uint32_t m = 0u - (uint32_t)alpha;
            auto pick = [&](float lo, float hi) {
                float r;
                asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(hi), "v"(lo));
                return r;
            };
            return make_pair_tab(s * pick(tv.v0, tv.v4), s * pick(tv.v1, tv.v5), s * pick(tv.v2, tv.v6),
                                 s * pick(tv.v3, tv.v7));
        };
        if constexpr (!PAIR_SHIFT) {
            PairTab t{0u, 0u};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (FMT == IQK_IQ2_K || (i & 1) == 0) t = table_of(i);  // IQ2_KS: one table per two code words
                u32x4 f0, f1;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    // bytes of v2: twice the codes of weights jj, 4 + jj, 8 + jj, 12 + jj
                    const uint32_t v2 = (jj == 0 ? q[i] << 1 : q[i] >> (2 * jj - 1)) & 0x06060606u;
                    const uint32_t v2p = v2 | 0x01010101u;
                    f0[jj] = pair_lookup(t, v2, v2p, sel_pair(0, 2));  // (jj, 8 + jj)
                    f1[jj] = pair_lookup(t, v2, v2p, sel_pair(1, 3));  // (4 + jj, 12 + jj)
                }
                emit(2 * i, f0);
                emit(2 * i + 1, f1);
            }
        } else {
#pragma unroll
            for (int ip = 0; ip < 4; ip += 2) {
                // the codes of two words shifted together: one 64-bit shift per
                // step (bits crossing from the high word into the low one land
                // outside the 0x06 mask of every byte)
                const uint64_t qq = ((uint64_t)q[ip + 1] << 32) | q[ip];
                uint32_t lo[4], hi[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    uint64_t sq;
                    if (jj == 0) asm("v_lshlrev_b64 %0, 1, %1" : "=v"(sq) : "v"(qq));
                    else asm("v_lshrrev_b64 %0, %1, %2" : "=v"(sq) : "i"(2 * jj - 1), "v"(qq));
                    lo[jj] = (uint32_t)sq;
                    hi[jj] = (uint32_t)(sq >> 32);
                }
                PairTab t = table_of(ip);  // IQ2_KS: one table for both words
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    const int i = ip + h2;
                    if (FMT == IQK_IQ2_K && h2 == 1) t = table_of(i);
                    u32x4 f0, f1;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        // bytes of v2: twice the codes of weights jj, 4 + jj, 8 + jj, 12 + jj
                        const uint32_t v2 = (h2 ? hi[jj] : lo[jj]) & 0x06060606u;
                        const uint32_t v2p = v2 | 0x01010101u;
                        f0[jj] = pair_lookup(t, v2, v2p, sel_pair(0, 2));  // (jj, 8 + jj)
                        f1[jj] = pair_lookup(t, v2, v2p, sel_pair(1, 3));  // (4 + jj, 12 + jj)
                    }
                    emit(2 * i, f0);
                    emit(2 * i + 1, f1);
                }
            }
        }
    } else {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const uint32_t h16 = (r.a >> (16 * b)) & 0xFFFFu;
            const float s = d * (float)(2 * ((h16 >> 12) & 7u) + 1);
            const float delta = (h16 >> 15) ? -0.125f : 0.125f;
            // entry 0: grid 0, 1: grid +1, 3: grid -1 (grid byte & 3)
            const PairTab t = make_pair_tab(s * delta, s * (1.0f + delta), 0.0f, s * (delta - 1.0f));
            const uint32_t qsw = b == 0 ? r.q.x : r.q.y;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t idx = ((qsw >> (8 * j)) & 0xFFu) | (((h16 >> (3 * j)) & 7u) << 8);
                const uint2 gv = grid_s[idx];  // doubled codes, staged that way
                const uint32_t v0p = gv.x | 0x01010101u, v1p = gv.y | 0x01010101u;
                u32x4 f;
                f[0] = pair_lookup(t, gv.x, v0p, sel_pair(0, 1));
                f[1] = pair_lookup(t, gv.x, v0p, sel_pair(2, 3));
                f[2] = pair_lookup(t, gv.y, v1p, sel_pair(0, 1));
                f[3] = pair_lookup(t, gv.y, v1p, sel_pair(2, 3));
                emit(4 * b + j, f);
            }
        }
    }
}

// Raw words of two adjacent 64-weight chunks c0, c0 + 1 (c0 even) of one
// row: the four lanes of a row then read its codes as one 128-byte line per
// 512 k instead of two half lines.
struct RowPair {
    uint4 q0, q1;
    uint32_t a, a2, b, c, d;
};

template <int FMT, int N>
__device__ __forceinline__ RowPair load_pair(const ExpertRes& x, uint32_t row, uint32_t c0) {
    using St = Strides<FMT, N>;
    RowPair r;
    r.a2 = r.c = 0;
    if constexpr (FMT == IQK_IQ2_K) {
        r.q0 = ld128(x.q, row * St::QS + 16u * c0);
        r.q1 = ld128(x.q, row * St::QS + 16u * c0 + 16u);
        r.a = ld32(x.a, row * St::P1 + 2u * c0);          // 4 scale nibbles per chunk
        r.b = ld8(x.b, row * St::P2 + (c0 >> 1));          // alphabet bits of both chunks
        r.d = ld16(x.d, row * St::P3 + 2u * (c0 >> 2));    // both chunks in one super-block
    } else if constexpr (FMT == IQK_IQ2_KS) {
        r.q0 = ld128(x.q, row * St::QS + 16u * c0);
        r.q1 = ld128(x.q, row * St::QS + 16u * c0 + 16u);
        r.a = ld16(x.a, row * St::P1 + c0);
        r.b = ld8(x.b, row * St::P2 + (c0 >> 2));
        r.c = ld8(x.c, row * St::P3 + (c0 >> 2));
        r.d = ld16(x.d, row * 2u);
    } else {
        const uint4 qq = ld128(x.q, row * St::QS + 8u * c0);
        r.q0 = make_uint4(qq.x, qq.y, 0u, 0u);
        r.q1 = make_uint4(qq.z, qq.w, 0u, 0u);
        const uint2 h = ld64(x.a, row * St::P1 + 4u * c0);
        r.a = h.x;
        r.a2 = h.y;
        r.b = 0;
        r.d = ld16(x.d, row * 2u);
    }
    return r;
}

// The words of chunk c0 + H of a pair in the single-chunk form.
template <int FMT, int H>
__device__ __forceinline__ RowData half_of(const RowPair& r) {
    RowData o;
    o.q = H ? r.q1 : r.q0;
    if constexpr (FMT == IQK_IQ2_K) o.a = H ? r.a >> 16 : r.a & 0xFFFFu;
    else if constexpr (FMT == IQK_IQ2_KS) o.a = H ? r.a >> 8 : r.a & 0xFFu;
    else o.a = H ? r.a2 : r.a;
    o.b = r.b;
    o.c = r.c;
    o.d = r.d;
    return o;
}

template <int FMT, int N>
struct FusedShared {
    __attribute__((aligned(16))) uint8_t A[kFStageBytes];  // token rows, fragment k order
    uint2 grid[FMT == IQK_IQ1_S_R4 ? 2048 : 1];
    float tab[8];
    int64_t xoff[16 * kFMT];  // element offset of each staged token row in x (-1: none)
};

// Fragment order of the staged token rows.  A super-step covers 512 k; lane
// group g owns chunks 2g and 2g + 1 of it (logical k 128 g .. 128 g + 127),
// and its step h (0, 1) uses chunk 2g + h.  Slot (h, mi, g, e) -- MFMA mi of
// step h, lane group g, element e -- sits at ((h * 8 + mi) * 4 + g) * 8 + e
// and holds logical k 128 g + 64 h + w(mi, e), w the within-chunk order of
// the fragment build (2-bit members: 16 (mi / 2) + 4 (mi % 2) + e / 2 +
// 8 (e % 2); IQ1_S_R4: 8 mi + e).

// Stage token rows tb .. tb + 16 MT of the expert (zeros past M) for k in
// [kc, kc + KC) into LDS in fragment order.  One unit = 16 logical k of one
// token row = two 16-byte slots; the loop is unrolled so every thread's
// loads are in flight together.  Row offsets come from sh.xoff.
template <int FMT, int N, int MT, int KC>
__device__ __forceinline__ void stage_tokens(const FusedParams& p, FusedShared<FMT, N>& sh, int kc, int tid) {
    constexpr int PITCH = 2 * KC + kFPad;
    constexpr int UNITS = 16 * MT * (KC / 16);
    constexpr int UPT = (UNITS + kFThreads - 1) / kFThreads;
#pragma unroll
    for (int it = 0; it < UPT; ++it) {
        const int u = tid + it * kFThreads;
        if (UNITS % kFThreads != 0 && u >= UNITS) break;
        const int r = u / (KC / 16);
        const int lu = u - r * (KC / 16);
        const int64_t xo = sh.xoff[r];
        uint32_t in[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
        if (xo >= 0) {
            const uint4* src = (const uint4*)(p.x + xo + kc + 16 * lu);
            const uint4 a = src[0], b = src[1];
            in[0] = a.x; in[1] = a.y; in[2] = a.z; in[3] = a.w;
            in[4] = b.x; in[5] = b.y; in[6] = b.z; in[7] = b.w;
        }
        const int L = (16 * lu) & 511;  // logical k inside the super-step
        const int sstep = (16 * lu) >> 9;
        const int gg = L >> 7;
        const int hh = (L >> 6) & 1;
        uint8_t* rowp = sh.A + r * PITCH + sstep * 1024;
        if constexpr (FMT == IQK_IQ1_S_R4) {
            const int mi = (L & 63) >> 3;  // two consecutive 8-weight groups
            *(uint4*)(rowp + (((hh * 8 + mi) * 4 + gg) * 8) * 2) = make_uint4(in[0], in[1], in[2], in[3]);
            *(uint4*)(rowp + (((hh * 8 + mi + 1) * 4 + gg) * 8) * 2) = make_uint4(in[4], in[5], in[6], in[7]);
        } else {
            const int i = (L & 63) >> 4;  // code word of the chunk
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t o[4];
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    // (L[4h + d], L[4h + d + 8]) from dwords holding (L[2w], L[2w + 1])
                    const int x = 4 * h + d;
                    o[d] = __builtin_amdgcn_perm(in[(x + 8) >> 1], in[x >> 1], (x & 1) ? 0x07060302u : 0x05040100u);
                }
                *(uint4*)(rowp + (((hh * 8 + 2 * i + h) * 4 + gg) * 8) * 2) = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    }
}

// Token tiles tb .. tb + 16 * MT of the expert against its row blocks
// rb0 .. rb1 - 1 (256 rows each; wave w owns rows 16 w .. 16 w + 15 of a
// block).  When all of k fits in LDS (one tile, or a short k) the tokens
// are staged once and the raw-word stream runs on from one row block into
// the next; otherwise each row block re-stages them 2048 k at a time.
template <int FMT, int N, int MT>
__device__ __forceinline__ void fused_pass(const FusedParams& p, FusedShared<FMT, N>& sh, const ExpertRes& res,
                                           const Table8& tv, int base, int M, int tb,
                                           int rb0, int rb1, int tid, int li, int g, int wave, bool nan_out) {
    constexpr int KC = MT == 1 ? (N < kFKC1 ? N : kFKC1) : (N < 2048 ? N : 2048);
    constexpr bool kPairShift = FMT == IQK_IQ2_KS || N <= 2048;
    constexpr int PITCH = 2 * KC + kFPad;  // LDS row pitch
    constexpr int SSC = KC / 512;          // super-steps per chunk
    // super-steps in flight (IQ2_KS: one, since two spill at k = 4096)
    constexpr int DW = FMT == IQK_IQ2_KS ? 1 : 2;
    constexpr int D = SSC < DW ? SSC : DW;
    constexpr bool WHOLE = KC == N;
    static_assert(MT * 16 * PITCH <= kFStageBytes && SSC % D == 0 && KC % 512 == 0, "staging layout");
    auto row_of = [&](int rb) __attribute__((always_inline)) { return rb * kFRows + wave * 16 + li; };
    const Rsrc yres = make_rsrc(p.y, (uint32_t)p.y_bytes);

    // D[token 4 g + i][weight row li] of each tile; absent tokens and rows
    // past `out` go to an out-of-range offset
    auto store = [&](const f32x4 (&acc)[MT], int row) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ti = tb + 16 * m + 4 * g + i;
                const bool ok = ti < M && row < p.out;
                const int pr = p.perm[base + (ok ? ti : 0)];
                __builtin_amdgcn_raw_buffer_store_b32(nan_out ? 0x7FC00000u : __float_as_uint(acc[m][i]), yres,
                                                      ok ? (uint32_t)((pr * p.out + row) * 4) : kOob, 0, 0);
            }
        }
    };
    auto mma_step = [&](f32x4 (&acc)[MT], const RowPair& rp, int c0, int sstep) __attribute__((always_inline)) {
        const uint8_t* arow = sh.A + li * PITCH + sstep * 1024 + g * 16;
        auto mma = [&](const uint8_t* ar, int mi, const u32x4& b) __attribute__((always_inline)) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const u32x4 a = *(const u32x4*)(ar + m * 16 * PITCH + mi * 64);
                acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                                 __builtin_bit_cast(bf16x8, b), acc[m], 0, 0, 0);
            }
        };
        decode_chunk<FMT, kPairShift>(half_of<FMT, 0>(rp), c0, tv, sh.grid, [&](int mi, const u32x4& b) __attribute__((always_inline)) { mma(arow, mi, b); });
        // IQ1_S_R4: keep the scheduler from hoisting the second half's grid
        // and activation reads over the first half (it runs out of registers)
        if constexpr (FMT == IQK_IQ1_S_R4 && N != 4096) __builtin_amdgcn_sched_barrier(0);
        decode_chunk<FMT, kPairShift>(half_of<FMT, 1>(rp), c0 + 1, tv, sh.grid,
                          [&](int mi, const u32x4& b) __attribute__((always_inline)) { mma(arow + 512, mi, b); });
    };
    auto write_xoff = [&]() __attribute__((always_inline)) {
        // the staged rows' activation offsets (the routing lookups once per row)
        if (tid < 16 * MT) {
            const int ti = tb + tid;
            int64_t off = -1;
            if (ti < M) {
                const int pair = p.perm[base + ti];
                const int t = pair / p.k;
                const int sl = p.x_slots == 1 ? 0 : pair - t * p.k;
                off = ((int64_t)t * p.x_slots + sl) * N;
            }
            sh.xoff[tid] = off;
        }
    };

    if constexpr (WHOLE) {
        RowPair buf[D];
#pragma unroll
        for (int u = 0; u < D; ++u) buf[u] = load_pair<FMT, N>(res, (uint32_t)row_of(rb0), (uint32_t)(8 * u + 2 * g));
        write_xoff();
        lds_barrier();  // offsets written; the previous pass's fragments are read
        stage_tokens<FMT, N, MT, KC>(p, sh, 0, tid);
        lds_barrier();
#pragma unroll 1
        for (int rb = rb0; rb < rb1; ++rb) {
            f32x4 acc[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
            for (int ss = 0; ss < SSC; ss += D) {
#pragma unroll
                for (int u = 0; u < D; ++u) {
                    mma_step(acc, buf[u], 8 * (ss + u) + 2 * g, ss + u);
                    // refill D super-steps ahead, running on into the next row block
                    const bool wrap = ss + u + D >= SSC;
                    const int nrb = wrap ? rb + 1 : rb;
                    const int nss = wrap ? ss + u + D - SSC : ss + u + D;
                    // (past the block's last row block: row `out`, out of range, reads zeros)
                    buf[u] = load_pair<FMT, N>(res, (uint32_t)(nrb < rb1 ? row_of(nrb) : p.out),
                                               (uint32_t)(8 * nss + 2 * g));
                }
            }
            store(acc, row_of(rb));
        }
    } else {
        write_xoff();
#pragma unroll 1
        for (int rb = rb0; rb < rb1; ++rb) {
            const int row = row_of(rb);
            f32x4 acc[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int kc = 0; kc < N; kc += KC) {
                // raw words of the chunk's first D super-steps, in flight during the staging
                RowPair buf[D];
#pragma unroll
                for (int u = 0; u < D; ++u)
                    buf[u] = load_pair<FMT, N>(res, (uint32_t)row, (uint32_t)(kc / 64 + 8 * u + 2 * g));
                lds_barrier();  // the previous chunk's fragments are read
                stage_tokens<FMT, N, MT, KC>(p, sh, kc, tid);
                lds_barrier();
#pragma unroll 1
                for (int ss = 0; ss < SSC; ss += D) {
#pragma unroll
                    for (int u = 0; u < D; ++u) {
                        const int c0 = kc / 64 + 8 * (ss + u) + 2 * g;
                        mma_step(acc, buf[u], c0, ss + u);
                        buf[u] = load_pair<FMT, N>(res, (uint32_t)(ss + u + D < SSC ? row : p.out),
                                                   (uint32_t)(c0 + 8 * D));
                    }
                }
            }
            store(acc, row);
        }
    }
}

// Work plan.  The kernel's work is split into units of one 256-row block of
// one expert; a unit's cost is the sum over the expert's token tiles of the
// measured cost of one pass (decode of the block's weights plus the MFMA
// work of 16 or 32 tokens; a 32-token pass over a 4096-wide row also
// re-stages its tokens per row block).  plan[e] is the cost of all units of
// experts before e; block b of G takes the units whose cost range starts in
// [b C / G, (b + 1) C / G), C = plan[E], so heavy experts are spread over
// more blocks and each block walks a contiguous run of row blocks.
template <int N>
__device__ __forceinline__ int64_t rb_cost(int M) {
    constexpr int C1 = 7;                  // one 16-token pass
    constexpr int C2 = N > 2048 ? 12 : 10;  // one 32-token pass
    const int full = M / 32, r = M - 32 * full;
    return (int64_t)full * C2 + (r > 16 ? C2 : (r > 0 ? C1 : 0));
}

template <int N>
__global__ __launch_bounds__(kFThreads) void fused_plan_kernel(const int32_t* offsets, int E, int nrb, int64_t* plan) {
    __shared__ int64_t part[kFThreads];
    const int tid = threadIdx.x;
    int64_t carry = 0;
    if (tid == 0) plan[0] = 0;
    for (int c = 0; c < E; c += kFThreads) {
        const int e = c + tid;
        const int64_t v = e < E ? rb_cost<N>(offsets[e + 1] - offsets[e]) * nrb : 0;
        part[tid] = v;
        __syncthreads();
        // inclusive scan (Hillis-Steele) over the chunk
        for (int o = 1; o < kFThreads; o <<= 1) {
            const int64_t add = tid >= o ? part[tid - o] : 0;
            __syncthreads();
            part[tid] += add;
            __syncthreads();
        }
        if (e < E) plan[e + 1] = carry + part[tid];
        carry += part[kFThreads - 1];
        __syncthreads();
    }
}

template <int FMT, int N>
__global__ __launch_bounds__(kFThreads) void fused_prefill_kernel(FusedParams p) {
    __shared__ FusedShared<FMT, N> sh;
    __shared__ int e_first;
    __shared__ uint64_t cand;            // experts e0 .. e0 + 63 with units in this block
    __shared__ int cand_rb[64][2];
    __shared__ int more;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int li = lane & 15;  // weight row of the tile (B) / token of the tile (A)
    const int g = lane >> 4;   // lane group: 128-weight span of the super-step
    const int nrb = (p.out + kFRows - 1) / kFRows;
    const int64_t C = p.plan[p.E];
    const int64_t lo = C * blockIdx.x / gridDim.x, hi = C * (blockIdx.x + 1) / gridDim.x;
    if (lo >= hi) return;

    uint32_t off_grid = 0;
    if constexpr (FMT == IQK_IQ1_S_R4) {
        // staged as doubled codes (2 (g & 3) per byte: the byte offset of
        // the grid value's bf16 in a pair table)
        for (int i = tid; i < 1024; i += kFThreads) {
            const uint4 v = ((const uint4*)p.grid)[i];
            ((uint4*)sh.grid)[i] = make_uint4((v.x & 0x03030303u) << 1, (v.y & 0x03030303u) << 1,
                                              (v.z & 0x03030303u) << 1, (v.w & 0x03030303u) << 1);
            off_grid |= non_ternary(v.x) | non_ternary(v.y) | non_ternary(v.z) | non_ternary(v.w);
        }
    }
    if (tid < 8) sh.tab[tid] = p.tab[tid];
    // the expert whose cost range holds lo (exactly one: plan is non-decreasing, plan[0] = 0 <= lo < C)
    for (int e = tid; e < p.E; e += kFThreads)
        if (p.plan[e] <= lo && p.plan[e + 1] > lo) e_first = e;
    // a grid value outside {-1, 0, +1}: every output of the block is NaN
    const bool nan_out = __syncthreads_or(off_grid != 0) != 0;
    // the value table in vector registers (the alphabet select needs them there)
    const Table8 tv{sh.tab[0], sh.tab[1], sh.tab[2], sh.tab[3], sh.tab[4], sh.tab[5], sh.tab[6], sh.tab[7]};

    for (int e0 = e_first;; e0 += 64) {
        if (wave == 0) {
            // row blocks rb of expert e whose cost range starts in [lo, hi)
            const int e = e0 + lane;
            int rb0 = 0, rb1 = 0;
            if (e < p.E) {
                const int64_t a = p.plan[e];
                const int64_t cr = rb_cost<N>(p.offsets[e + 1] - p.offsets[e]);
                if (cr > 0 && a < hi) {
                    const int64_t s0 = lo > a ? (lo - a + cr - 1) / cr : 0;
                    const int64_t s1 = (hi - a + cr - 1) / cr;
                    rb0 = (int)s0;
                    rb1 = (int)(s1 < nrb ? s1 : nrb);
                }
            }
            cand_rb[lane][0] = rb0;
            cand_rb[lane][1] = rb1;
            const uint64_t m = __ballot(rb0 < rb1);
            if (lane == 0) {
                cand = m;
                more = e0 + 64 < p.E && p.plan[e0 + 64] < hi;
            }
        }
        __syncthreads();
        uint64_t m = cand;
        const int go_on = more;
        while (m) {
            const int j = __builtin_ctzll(m);
            m &= m - 1;
            const int e = e0 + j;
            const int rb0 = cand_rb[j][0], rb1 = cand_rb[j][1];
            const int base = p.offsets[e];
            const int M = p.offsets[e + 1] - base;
            const ExpertRes res = expert_res<FMT, N>(p, e);
            for (int tb = 0; tb < M; tb += 16 * kFMT) {
                if (M - tb > 16) fused_pass<FMT, N, 2>(p, sh, res, tv, base, M, tb, rb0, rb1, tid, li, g, wave, nan_out);
                else fused_pass<FMT, N, 1>(p, sh, res, tv, base, M, tb, rb0, rb1, tid, li, g, wave, nan_out);
            }
        }
        if (!go_on) break;
        __syncthreads();  // every wave has read cand before wave 0 rewrites it
    }
}

int fused_grid_blocks() {
    // one block per compute unit (a block's LDS leaves room for no second one)
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

template <int FMT, int N>
hipError_t launch_fused_n(const FusedParams& p, const int32_t* offsets, int64_t* plan, hipStream_t s) {
    const int nrb = (p.out + kFRows - 1) / kFRows;
    hipLaunchKernelGGL((fused_plan_kernel<N>), dim3(1), dim3(kFThreads), 0, s, offsets, p.E, nrb, plan);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((fused_prefill_kernel<FMT, N>), dim3((unsigned)fused_grid_blocks()), dim3(kFThreads), 0, s, p);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_fused_fmt(const FusedParams& p, int64_t n, const int32_t* offsets, int64_t* plan, hipStream_t s) {
    if (n == 4096) return launch_fused_n<FMT, 4096>(p, offsets, plan, s);
    if (n == 2048) return launch_fused_n<FMT, 2048>(p, offsets, plan, s);
    return launch_fused_n<FMT, 512>(p, offsets, plan, s);
}

}  // namespace

hipError_t launch_fused_prefill(const FusedLaunch& a, hipStream_t s) {
    FusedParams p;
    p.S = a.streams;
    p.off0 = a.pl.off[0];
    p.off1 = a.pl.off[1];
    p.off2 = a.pl.off[2];
    p.off3 = a.pl.off[3];
    p.off4 = a.pl.off[4];
    p.E = (int32_t)a.E;
    p.out = (int32_t)a.out;
    for (int i = 0; i < 8; ++i) p.tab[i] = a.values ? a.values[i] : 0.f;
    p.grid = a.grid;
    p.x = (const uint16_t*)a.x;
    p.x_slots = a.x_slots;
    p.k = a.k;
    p.offsets = a.offsets;
    p.perm = a.perm;
    p.y = a.y;
    p.y_bytes = a.T * a.k * a.out * 4;
    p.plan = a.plan;
    if (a.fmt == IQK_IQ2_KS) return launch_fused_fmt<IQK_IQ2_KS>(p, a.n, a.offsets, a.plan, s);
    if (a.fmt == IQK_IQ2_K) return launch_fused_fmt<IQK_IQ2_K>(p, a.n, a.offsets, a.plan, s);
    return launch_fused_fmt<IQK_IQ1_S_R4>(p, a.n, a.offsets, a.plan, s);
}

}  // namespace iqk
