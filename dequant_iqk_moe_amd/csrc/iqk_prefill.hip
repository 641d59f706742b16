// iqk_prefill.hip -- routing gather and the MFMA grouped GEMM of prefill.
//
// "mlx-iqk" package description, "Surface": a call with many token-expert
// pairs dequantizes the stacked experts and runs a grouped GEMM (MLX's
// gather_mm), honouring the caller's sort flag so that each expert's
// weights are read once per sorted prefill.
//
// Routing: one workgroup builds per-expert counts (LDS atomics), an
// exclusive scan, and a stable expert-major permutation of the pairs; the
// stable scatter ranks 64 pairs at a time per wave, equal ids found with
// ballots, so the order inside an expert is the pair order.  When the caller
// states that the ids are sorted and the histogram pass confirms they are
// non-decreasing, the stable sort is the identity on the valid pairs and the
// ranking is skipped.  Pairs with an id outside [0, E) are dropped; when the
// caller passes its output, their rows are set to NaN here (the prefill and
// grouped kernels only write the rows of routed pairs).
//
// Grouped GEMM: per expert e with M_e routed pairs, Y_e = X_e W_e^T with bf16
// inputs and float32 accumulation on v_mfma_f32_16x16x32_bf16.  A workgroup
// owns one expert and 256 weight rows (4 waves x 64 rows); each wave keeps
// up to kMT 16-token tiles of accumulators so its weight rows are streamed
// from HBM once for up to 16*kMT tokens.  Token rows are gathered straight
// from x through the permutation (no gather copy) and results are scattered
// straight to y[t, j, :] (no scatter pass).  Operands are loaded from global
// memory directly into MFMA registers: both operands use the same k order
// (lane group g takes k = 16g..16g+15 of each 64-wide step, split over two
// MFMAs), so every 16-byte load is part of a full 128-byte line per row.
#include "iqk_internal.h"

namespace iqk {
namespace {

// ---------------------------------------------------------------------------
// routing gather
// ---------------------------------------------------------------------------

constexpr int kRouteThreads = 1024;
constexpr int kRouteMaxE = 16384;
constexpr int kRouteStage = 4096;  // ids staged in LDS per scatter chunk
constexpr int kRouteWaves = kRouteThreads / 64;
constexpr int kRouteHistE = 1024;  // experts up to which the waves rank in parallel

__global__ __launch_bounds__(kRouteThreads) void route_kernel(const int32_t* __restrict__ ids, int32_t P, int32_t E,
                                                              int32_t sorted, int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ perm, float* __restrict__ ynan,
                                                              int32_t yout) {
    __shared__ int32_t cur[kRouteMaxE];
    __shared__ int32_t part[kRouteThreads];
    __shared__ int32_t stage[kRouteStage];
    __shared__ int32_t hist[kRouteWaves * kRouteHistE];  // per-wave expert counts, then starts
    __shared__ int32_t n_bad, n_neg;                      // invalid ids, ids below zero
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kRouteThreads) cur[e] = 0;
    if (tid == 0) n_bad = n_neg = 0;
    __syncthreads();
    int descents = 0;  // ids[p - 1] > ids[p] seen by this thread (checked only for a sorted call)
    for (int p = tid; p < P; p += kRouteThreads) {
        const int e = ids[p];
        if (e >= 0 && e < E) {
            atomicAdd(&cur[e], 1);
        } else {
            atomicAdd(&n_bad, 1);
            if (e < 0) atomicAdd(&n_neg, 1);
        }
        if (sorted && p > 0 && ids[p - 1] > e) descents = 1;
    }
    // (the barrier after the histogram, taken by every thread whatever the flag)
    const bool any_descent = __syncthreads_or(descents) != 0;
    const bool identity = sorted && !any_descent;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    if (ynan && n_bad > 0) {
        // NaN rows for the dropped pairs, one wave per pair
        for (int p0 = wave * 64; p0 < P; p0 += kRouteThreads) {
            const int e = p0 + lane < P ? ids[p0 + lane] : 0;
            uint64_t m = __ballot(e < 0 || e >= E);
            while (m) {
                const int pp = p0 + __builtin_ctzll(m);
                m &= m - 1;
                float* row = ynan + (int64_t)pp * yout;
                for (int o = lane; o < yout; o += 64) row[o] = __builtin_nanf("");
            }
        }
    }
    // exclusive scan: each thread owns a contiguous segment of experts
    const int seg = (E + kRouteThreads - 1) / kRouteThreads;
    const int e0 = min(tid * seg, E), e1 = min(e0 + seg, E);
    int s = 0;
    for (int e = e0; e < e1; ++e) s += cur[e];
    part[tid] = s;
    __syncthreads();
    for (int d = 1; d < kRouteThreads; d <<= 1) {  // Hillis-Steele inclusive scan of segment sums
        const int v = tid >= d ? part[tid - d] : 0;
        __syncthreads();
        part[tid] += v;
        __syncthreads();
    }
    int run = part[tid] - s;
    for (int e = e0; e < e1; ++e) {
        const int c = cur[e];
        counts[e] = c;
        offsets[e] = run;
        cur[e] = run;
        run += c;
    }
    if (tid == kRouteThreads - 1) offsets[E] = part[tid];
    const int total = part[kRouteThreads - 1];
    // positions past the valid pairs (invalid ids are dropped)
    for (int p = total + tid; p < P; p += kRouteThreads) perm[p] = -1;
    if (identity) {
        // non-decreasing ids: ids below zero come first, ids >= E last, and
        // the valid pairs in between are already in stable expert order
        const int first = n_neg;
        for (int i = tid; i < total; i += kRouteThreads) perm[i] = first + i;
        return;
    }
    // stable scatter.  The ids are staged in LDS a chunk at a time.  Up to
    // kRouteHistE experts, each wave takes a contiguous slice of the chunk:
    // per-wave expert counts, an exclusive prefix over the waves gives each
    // wave its per-expert start, and the waves then rank their slices in
    // parallel.  Beyond that, one wave ranks the whole chunk.  Ranking: 64
    // pairs per step, equal ids found with one ballot per id bit.
    int nbits = 1;
    while ((1 << nbits) < E) ++nbits;
    const uint64_t lt = (1ull << lane) - 1ull;
    const bool waves_split = E <= kRouteHistE;
    // ranks the pairs [i0, i1) of the staged chunk against the cursors cur_w
    auto rank_slice = [&](int base, int i0, int i1, int32_t* cur_w) {
        for (int s0 = i0; s0 < i1; s0 += 64) {
            const int i = s0 + lane;
            const int e = i < i1 ? stage[i] : -1;
            const bool valid = e >= 0 && e < E;
            uint64_t same = __ballot(valid);
            for (int b = 0; b < nbits; ++b) {
                const bool bit = valid && ((e >> b) & 1);
                const uint64_t m = __ballot(bit);
                same &= bit ? m : ~m;
            }
            const int rank = __popcll(same & lt);
            const int cnt = __popcll(same);
            int pos = 0;
            if (valid) pos = cur_w[e] + rank;
            __builtin_amdgcn_wave_barrier();
            if (valid && rank == cnt - 1) cur_w[e] = pos + 1;  // last of its expert advances the cursor
            __builtin_amdgcn_wave_barrier();
            if (valid) perm[pos] = base + i;
        }
    };
    for (int base = 0; base < P; base += kRouteStage) {
        const int n = min(kRouteStage, P - base);
        __syncthreads();  // the cursors are final / the previous chunk is ranked
        for (int i = tid; i < n; i += kRouteThreads) stage[i] = ids[base + i];
        if (waves_split)
            for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) hist[i] = 0;
        __syncthreads();
        if (waves_split) {
            const int per = (n + kRouteWaves - 1) / kRouteWaves;
            const int i0 = min(wave * per, n), i1 = min(i0 + per, n);
            for (int i = i0 + lane; i < i1; i += 64) {
                const int e = stage[i];
                if (e >= 0 && e < E) atomicAdd(&hist[wave * E + e], 1);
            }
            __syncthreads();
            // hist[w][e] <- start of wave w's pairs of expert e; cur[e] advances past the chunk
            for (int e = tid; e < E; e += kRouteThreads) {
                int run = cur[e];
                for (int w = 0; w < kRouteWaves; ++w) {
                    const int c = hist[w * E + e];
                    hist[w * E + e] = run;
                    run += c;
                }
                cur[e] = run;
            }
            __syncthreads();
            rank_slice(base, i0, i1, hist + wave * E);
        } else if (tid < 64) {
            rank_slice(base, 0, n, cur);
        }
    }
}

// ---------------------------------------------------------------------------
// grouped GEMM
// ---------------------------------------------------------------------------

constexpr int kGemmWaves = 4;
constexpr int kGemmThreads = 64 * kGemmWaves;
constexpr int kRowsPerWave = 64;                       // 4 MFMA column tiles of 16 weight rows
constexpr int kRowsPerWG = kRowsPerWave * kGemmWaves;  // 256
constexpr int kMT = 2;                                 // 16-token tiles held per wave

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct GemmParams {
    const uint16_t* W;
    int32_t E, out, n;
    const uint16_t* x;
    int32_t x_slots, k;
    const int32_t* offsets;
    const int32_t* perm;
    float* y;
};

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__global__ __launch_bounds__(kGemmThreads) void grouped_gemm_kernel(GemmParams p) {
    const int e = blockIdx.y;
    const int row_wg = blockIdx.x * kRowsPerWG;
    const int begin = p.offsets[e];
    const int M = p.offsets[e + 1] - begin;
    if (M <= 0) return;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int row0 = row_wg + wave * kRowsPerWave;
    if (row0 >= p.out) return;
    const int li = lane & 15;   // token (A) / weight row (B) inside a 16-tile
    const int kg = lane >> 4;   // k group
    const int n = p.n;

    // weight rows of this lane, one per column tile (tiles past `out` idle)
    const uint16_t* wrow[4];
    bool cvalid[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        cvalid[c] = row0 + 16 * c < p.out;
        wrow[c] = p.W + ((int64_t)e * p.out + (cvalid[c] ? row0 + 16 * c + li : 0)) * n + 16 * kg;
    }

    for (int mbase = 0; mbase < M; mbase += 16 * kMT) {
        const uint16_t* xrow[kMT];
        int pair_of[kMT];
#pragma unroll
        for (int m = 0; m < kMT; ++m) {
            const int idx = mbase + 16 * m + li;
            pair_of[m] = idx < M ? p.perm[begin + idx] : -1;
            if (pair_of[m] >= 0) {
                const int t = pair_of[m] / p.k;
                const int s = p.x_slots == 1 ? 0 : pair_of[m] - t * p.k;
                xrow[m] = p.x + ((int64_t)t * p.x_slots + s) * n + 16 * kg;
            } else {
                xrow[m] = nullptr;
            }
        }
        f32x4 acc[kMT][4];
#pragma unroll
        for (int m = 0; m < kMT; ++m)
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[m][c] = f32x4{0.f, 0.f, 0.f, 0.f};

        for (int k0 = 0; k0 < n; k0 += 64) {
            u32x4 b[4][2], a[kMT][2];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (cvalid[c]) {
                    const u32x4* src = (const u32x4*)(wrow[c] + k0);
                    b[c][0] = __builtin_nontemporal_load(src);
                    b[c][1] = __builtin_nontemporal_load(src + 1);
                } else {
                    b[c][0] = b[c][1] = u32x4{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int m = 0; m < kMT; ++m) {
                if (xrow[m]) {
                    const u32x4* src = (const u32x4*)(xrow[m] + k0);
                    a[m][0] = src[0];
                    a[m][1] = src[1];
                } else {
                    a[m][0] = a[m][1] = u32x4{0u, 0u, 0u, 0u};
                }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int m = 0; m < kMT; ++m)
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        acc[m][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[m][h]), as_bf16x8(b[c][h]),
                                                                            acc[m][c], 0, 0, 0);
        }
        // D[token 4*kg + i][weight row li] of each tile
#pragma unroll
        for (int m = 0; m < kMT; ++m) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = 4 * kg + i;
                const int pr = __shfl(pair_of[m], tok);  // pair of token row `tok` lives in lane tok
                if (pr >= 0) {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (cvalid[c]) p.y[(int64_t)pr * p.out + row0 + 16 * c + li] = acc[m][c][i];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// plain streaming read (HBM floor-rate reference)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ buf, int64_t n16, uint32_t* sink,
                                                          int64_t sink_words) {
    uint32_t acc = 0;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(buf + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o);
    // any lane's value will do; plain stores, the sink only keeps the loads alive
    if ((threadIdx.x & 63) == 0) sink[((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) % sink_words] = acc;
}

// plain streaming write (HBM write-ceiling reference): the value in every
// 16-byte word, non-temporal 16-byte stores, a wave covering 1 KiB per store
// instruction; each wave writes `runs` consecutive 1 KiB runs, the waves of
// a workgroup adjacent spans.  One run per wave is the fastest plain write
// measured on this part (6.7 TB/s over 8.6 GB, against 5.3-5.9 TB/s for
// eight or more stores per wave in any order tried); eight runs per wave is
// the store shape of the bf16 dequantization producer.
__global__ __launch_bounds__(256) void stream_write_kernel(u32x4* __restrict__ buf, int64_t n16, int runs,
                                                           uint32_t value) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t w0 = ((int64_t)blockIdx.x * 4 + wave) * runs * 64;
    const u32x4 v = {value, value, value, value};
    for (int r = 0; r < runs; ++r) {
        const int64_t i = w0 + (int64_t)r * 64 + lane;
        if (i < n16) __builtin_nontemporal_store(v, buf + i);
    }
}

}  // namespace

hipError_t launch_stream_write(void* buf, size_t bytes, uint32_t value, int runs, hipStream_t s) {
    const int64_t n16 = (int64_t)(bytes / 16);
    const int64_t per_block = (int64_t)256 * runs;  // 16-byte words per workgroup
    const int64_t blocks = (n16 + per_block - 1) / per_block;
    if (blocks < 1 || blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    hipLaunchKernelGGL(stream_write_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (u32x4*)buf, n16, runs, value);
    return hipGetLastError();
}

hipError_t launch_route(const RouteLaunch& a, hipStream_t s) {
    if (a.E > kRouteMaxE) return hipErrorInvalidValue;
    hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kRouteThreads), 0, s, a.ids, (int32_t)a.P, (int32_t)a.E,
                       (int32_t)a.sorted, a.counts, a.offsets, a.perm, a.ynan, (int32_t)a.yout);
    return hipGetLastError();
}

hipError_t launch_grouped_gemm(const GemmLaunch& a, hipStream_t s) {
    GemmParams p;
    p.W = (const uint16_t*)a.W;
    p.E = (int32_t)a.E;
    p.out = (int32_t)a.out;
    p.n = (int32_t)a.n;
    p.x = (const uint16_t*)a.x;
    p.x_slots = a.x_slots;
    p.k = a.k;
    p.offsets = a.offsets;
    p.perm = a.perm;
    p.y = a.y;
    if (a.n % 64) return hipErrorInvalidValue;
    const unsigned gx = (unsigned)((a.out + kRowsPerWG - 1) / kRowsPerWG);
    hipLaunchKernelGGL(grouped_gemm_kernel, dim3(gx, (unsigned)a.E), dim3(kGemmThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words, hipStream_t s) {
    const int64_t n16 = (int64_t)(bytes / 16);
    int64_t blocks = (n16 + 255) / 256;
    blocks = blocks < 256 * 16 ? blocks : 256 * 16;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (const u32x4*)buf, n16, sink,
                       (int64_t)sink_words);
    return hipGetLastError();
}

}  // namespace iqk
