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
// table value, or d * float(2 ls + 1) * (grid value + shift), float32, then
// one round-to-nearest-even cast to bf16; every such product is exact in
// float32, so the order of the two multiplications does not matter).
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
//     of a fragment is then one v_perm_b32 of that table, its selector one
//     v_perm_b32 of doubled code bytes.  About 2-3 VALU instructions per
//     weight, once per weight whatever the number of tokens.
//   * The expert's token rows (gathered through the routing permutation)
//     are staged in LDS, 2048 k at a time for up to 32 tokens, already in
//     the k order the fragments use (a per-step permutation that makes both
//     the table lookups and the LDS reads 16-byte contiguous); rows are
//     padded by 16 bytes so a fragment read is bank-conflict free.
//   * Results go straight to y[t, j, :] (no scatter pass).
#include "iqk_device.h"

namespace iqk {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kFWaves = 16;                 // waves per block, one 16-row tile each
constexpr int kFThreads = 64 * kFWaves;
constexpr int kFRows = 16 * kFWaves;        // weight rows per block
constexpr int kFMT = 2;                     // 16-token tiles per pass over k
constexpr int kFKChunk = 2048;              // activation k staged in LDS at a time
constexpr int kFRowBytes = 2 * kFKChunk + 16;  // LDS row pitch (padding: conflict-free reads)

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

// Two bf16 weights from a 4-entry table (entries 0..3 at bytes 2c, 2c+1 of
// tlo:thi): `d2` holds 2 * code in its bytes, `d2p1` 2 * code + 1, and
// `sel` picks which two code bytes form the pair.
__device__ __forceinline__ uint32_t table_pair(uint32_t tlo, uint32_t thi, uint32_t d2, uint32_t d2p1, uint32_t sel) {
    return __builtin_amdgcn_perm(thi, tlo, __builtin_amdgcn_perm(d2p1, d2, sel));
}

// Fragment selectors: bytes (x, y) of the code word give the pair
// [2 c_x, 2 c_x + 1, 2 c_y, 2 c_y + 1] (byte 4 + i of the perm source is
// byte i of d2p1).
constexpr uint32_t sel_pair(int x, int y) {
    return (uint32_t)x | (uint32_t)(4 + x) << 8 | (uint32_t)y << 16 | (uint32_t)(4 + y) << 24;
}

// 4-entry bf16 table of one sub-block: values v0..v3.
struct Tab {
    uint32_t lo, hi;
};
__device__ __forceinline__ Tab make_tab(float v0, float v1, float v2, float v3) {
    return Tab{pk_bf16(v0, v1), pk_bf16(v2, v3)};
}

// The eight B fragments (4 dwords each) of one lane's 64-weight chunk.
// 2-bit members: fragment 2i + h holds weights (4h + d, 4h + d + 8) of code
// word i as dword d; IQ1_S_R4: fragment 2b + j holds group j of block b in
// natural order.
template <int FMT>
__device__ __forceinline__ void decode_chunk(const RowData& r, int c, const float* tab, const uint2* grid_s,
                                             u32x4 (&B)[8]) {
    const float d = half_to_float(r.d);
    if constexpr (FMT == IQK_IQ2_K || FMT == IQK_IQ2_KS) {
        const uint32_t q[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
        Tab t{0u, 0u};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int si;
            uint32_t alpha;
            if constexpr (FMT == IQK_IQ2_K) {
                si = __builtin_amdgcn_sbfe((int)(r.a ^ 0x8888u), 4 * i, 4);  // nibble - 8
                alpha = (r.b >> (4 * (c & 1) + i)) & 1u;
            } else {
                const int j = i >> 1;  // 32-weight sub-block
                const int sh = 2 * (c & 3) + j;
                si = (int)(((r.a >> (4 * j)) & 15u) | (((r.b >> sh) & 1u) << 4)) - 16;
                alpha = (r.c >> sh) & 1u;
            }
            if (FMT == IQK_IQ2_K || (i & 1) == 0) {  // IQ2_KS: one table per two code words
                const float s = d * (float)si;
                t = alpha ? make_tab(s * tab[4], s * tab[5], s * tab[6], s * tab[7])
                          : make_tab(s * tab[0], s * tab[1], s * tab[2], s * tab[3]);
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                // bytes of v: codes of weights jj, 4 + jj, 8 + jj, 12 + jj
                const uint32_t v = (q[i] >> (2 * jj)) & 0x03030303u;
                const uint32_t d2 = v + v, d2p1 = d2 + 0x01010101u;
                B[2 * i][jj] = table_pair(t.lo, t.hi, d2, d2p1, sel_pair(0, 2));      // (jj, 8 + jj)
                B[2 * i + 1][jj] = table_pair(t.lo, t.hi, d2, d2p1, sel_pair(1, 3));  // (4 + jj, 12 + jj)
            }
        }
    } else {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            const uint32_t h16 = (r.a >> (16 * b)) & 0xFFFFu;
            const float s = d * (float)(2 * ((h16 >> 12) & 7u) + 1);
            const float delta = (h16 >> 15) ? -0.125f : 0.125f;
            // entry 0: grid 0, 1: grid +1, 3: grid -1 (grid byte & 3)
            const Tab t = make_tab(s * delta, s * (1.0f + delta), 0.0f, s * (delta - 1.0f));
            const uint32_t qsw = b == 0 ? r.q.x : r.q.y;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t idx = ((qsw >> (8 * j)) & 0xFFu) | (((h16 >> (3 * j)) & 7u) << 8);
                const uint2 gv = grid_s[idx];
                const uint32_t v0 = gv.x & 0x03030303u, v1 = gv.y & 0x03030303u;
                const uint32_t a2 = v0 + v0, a2p1 = a2 + 0x01010101u;
                const uint32_t b2 = v1 + v1, b2p1 = b2 + 0x01010101u;
                B[4 * b + j][0] = table_pair(t.lo, t.hi, a2, a2p1, sel_pair(0, 1));
                B[4 * b + j][1] = table_pair(t.lo, t.hi, a2, a2p1, sel_pair(2, 3));
                B[4 * b + j][2] = table_pair(t.lo, t.hi, b2, b2p1, sel_pair(0, 1));
                B[4 * b + j][3] = table_pair(t.lo, t.hi, b2, b2p1, sel_pair(2, 3));
            }
        }
    }
}

// Logical k (inside a 256-wide step) of fragment slot pp = (mi * 4 + g) * 8 + e
// of MFMA mi, lane group g, element e: the k order both operands share.
template <int FMT>
__device__ __forceinline__ int slot_k(int mi, int g, int e) {
    if constexpr (FMT == IQK_IQ1_S_R4) return 64 * g + 8 * mi + e;
    return 64 * g + 16 * (mi >> 1) + 4 * (mi & 1) + (e >> 1) + 8 * (e & 1);
}

template <int FMT, int N>
__global__ __launch_bounds__(kFThreads) void fused_prefill_kernel(FusedParams p) {
    constexpr int KC = N < kFKChunk ? N : kFKChunk;
    __shared__ __attribute__((aligned(16))) uint8_t A_s[kFMT * 16 * kFRowBytes];
    __shared__ uint2 grid_s[FMT == IQK_IQ1_S_R4 ? 2048 : 1];

    const int e = blockIdx.y;
    const int base = p.offsets[e];
    const int M = p.offsets[e + 1] - base;
    if (M <= 0) return;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int li = lane & 15;  // weight row of the tile (B) / token of the tile (A)
    const int g = lane >> 4;   // lane group: 64-weight chunk of the step
    const int row = blockIdx.x * kFRows + wave * 16 + li;  // rows past `out` read zeros
    const ExpertRes res = expert_res<FMT, N>(p, e);
    const ExpertRes none = expert_res<FMT, N>(p, -1);  // zero records: reads nothing

    if constexpr (FMT == IQK_IQ1_S_R4) {
        ((uint4*)grid_s)[tid] = ((const uint4*)p.grid)[tid];  // 1024 x 16 bytes
    }

    for (int tb = 0; tb < M; tb += 16 * kFMT) {
        const int mtc = M - tb > 16 ? 2 : 1;  // token tiles in this pass
        f32x4 acc[kFMT];
#pragma unroll
        for (int m = 0; m < kFMT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int kc = 0; kc < N; kc += KC) {
            // this lane's first raw words of the chunk, in flight during the staging
            RowData cur = load_row<FMT, N>(res, (uint32_t)row, (uint32_t)(kc / 64 + g));
            lds_barrier();  // the previous chunk's fragments are read
            // Stage tokens tb .. tb + 32 (zeros past M) for k in [kc, kc + KC):
            // one unit = 16 logical k of one token row = two 16-byte slots.
            for (int u = tid; u < 16 * kFMT * (KC / 16); u += kFThreads) {
                const int r = u / (KC / 16);
                const int lu = u - r * (KC / 16);
                const int ti = tb + r;
                uint32_t in[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
                if (ti < M) {
                    const int pair = p.perm[base + ti];
                    const int t = pair / p.k;
                    const int sl = p.x_slots == 1 ? 0 : pair - t * p.k;
                    const uint4* src = (const uint4*)(p.x + ((int64_t)t * p.x_slots + sl) * N + kc + 16 * lu);
                    const uint4 a = src[0], b = src[1];
                    in[0] = a.x; in[1] = a.y; in[2] = a.z; in[3] = a.w;
                    in[4] = b.x; in[5] = b.y; in[6] = b.z; in[7] = b.w;
                }
                const int L = (16 * lu) & 255;  // logical k inside the step
                const int step = (16 * lu) >> 8;
                const int gg = L >> 6;
                uint8_t* rowp = A_s + r * kFRowBytes + step * 512;
                if constexpr (FMT == IQK_IQ1_S_R4) {
                    const int mi = (L & 63) >> 3;  // two consecutive 8-weight groups
                    *(uint4*)(rowp + ((mi * 4 + gg) * 8) * 2) = make_uint4(in[0], in[1], in[2], in[3]);
                    *(uint4*)(rowp + (((mi + 1) * 4 + gg) * 8) * 2) = make_uint4(in[4], in[5], in[6], in[7]);
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
                        *(uint4*)(rowp + (((2 * i + h) * 4 + gg) * 8) * 2) = make_uint4(o[0], o[1], o[2], o[3]);
                    }
                }
            }
            lds_barrier();

            // k steps of this chunk: raw words one step ahead (the step after
            // the chunk's last reads nothing)
            for (int st = 0; st < KC / 256; ++st) {
                const int c = (kc + 256 * st) / 64 + g;  // this lane's chunk
                const RowData nxt = load_row<FMT, N>(st + 1 < KC / 256 ? res : none, (uint32_t)row, (uint32_t)(c + 4));
                u32x4 B[8];
                decode_chunk<FMT>(cur, c, p.tab, grid_s, B);
#pragma unroll
                for (int mi = 0; mi < 8; ++mi) {
#pragma unroll
                    for (int m = 0; m < kFMT; ++m) {
                        if (m < mtc) {
                            const u32x4 a = *(const u32x4*)(A_s + (m * 16 + li) * kFRowBytes + st * 512 +
                                                            ((mi * 4 + g) * 8) * 2);
                            acc[m] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                                             __builtin_bit_cast(bf16x8, B[mi]),
                                                                             acc[m], 0, 0, 0);
                        }
                    }
                }
                cur = nxt;
            }
        }
        // D[token 4 g + i][weight row li]
        if (row < p.out) {
#pragma unroll
            for (int m = 0; m < kFMT; ++m) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int ti = tb + 16 * m + 4 * g + i;
                    if (m < mtc && ti < M) p.y[(int64_t)p.perm[base + ti] * p.out + row] = acc[m][i];
                }
            }
        }
    }
}

template <int FMT, int N>
hipError_t launch_fused_n(const FusedParams& p, hipStream_t s) {
    const unsigned gx = (unsigned)((p.out + kFRows - 1) / kFRows);
    hipLaunchKernelGGL((fused_prefill_kernel<FMT, N>), dim3(gx, (unsigned)p.E), dim3(kFThreads), 0, s, p);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_fused_fmt(const FusedParams& p, int64_t n, hipStream_t s) {
    if (n == 4096) return launch_fused_n<FMT, 4096>(p, s);
    if (n == 2048) return launch_fused_n<FMT, 2048>(p, s);
    return launch_fused_n<FMT, 512>(p, s);
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
    if (a.fmt == IQK_IQ2_KS) return launch_fused_fmt<IQK_IQ2_KS>(p, a.n, s);
    if (a.fmt == IQK_IQ2_K) return launch_fused_fmt<IQK_IQ2_K>(p, a.n, s);
    return launch_fused_fmt<IQK_IQ1_S_R4>(p, a.n, s);
}

}  // namespace iqk
