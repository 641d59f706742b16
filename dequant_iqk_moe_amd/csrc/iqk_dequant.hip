// iqk_dequant.hip -- dequantization of canonical IQ_K streams (the prefill
// weight producer).  "mlx-iqk" package description, "Format" section: every
// weight is rebuilt as a float32 chain in the CPU dequantizer's order,
//   2-bit:    w = (float(d) * float(scale_index)) * values[4*alphabet + code]
//   IQ1_S_R4: w = (float(d) * float(2*ls + 1)) * (float(grid_value) + shift)
// and, for half-precision outputs, rounded once to nearest-even.  The
// introduction states that the producer "dequantizes the stacked experts in
// one kernel pass" at the streaming floor.
//
// The path is write-bound (2 or 4 output bytes per 0.19-0.30 input bytes), so
// the design keeps every wave store a contiguous 1 KiB run: one item = 16
// output bytes (8 weights for f16/bf16, 4 for f32), consecutive lanes take
// consecutive items, and the grid strides over items.  Per-item field loads
// (a 2-byte code word, 1-byte scale/alphabet words, the fp16 scale) hit L1/L2
// after the first lane of a sub-block.  This file is compiled without FMA
// contraction; every multiply rounds on its own.
#include "iqk_internal.h"

namespace iqk {
namespace {

constexpr int kThreads = 256;
#ifndef IQK_DEQUANT_MAX_BLOCKS
#define IQK_DEQUANT_MAX_BLOCKS (256 * 512)
#endif
// IQ1_S_R4 workgroups stage the grid in LDS before their first chunk, so
// each thread walks at least this many chunks (measured: one chunk per
// thread, the shape of a [4096, 2048] projection under the plain cap, is 7 %
// slower than two or more)
#ifndef IQK_DEQUANT_GRID_CHUNKS
#define IQK_DEQUANT_GRID_CHUNKS 2
#endif

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void store16_nt(void* base, int64_t item, u32x4 v) {
    __builtin_nontemporal_store(v, (u32x4*)base + item);
}

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// One item = 16 bytes of output; W weights per item.
template <int OUT_DT>
struct ItemShape {
    static constexpr int W = OUT_DT == IQK_F32 ? 4 : 8;
};

// The float32 product must be rounded to float32 before the half cast; left
// alone, the compiler folds fptrunc(fmul) into v_fma_mix*_f16, which rounds
// the exact product once, straight to f16.  An empty asm pins the float32
// value in a VGPR.
__device__ __forceinline__ float pin_f32(float v) {
    asm volatile("" : "+v"(v));
    return v;
}

__device__ __forceinline__ uint32_t pack2(float a, float b, int out_dt) {
    if (out_dt == IQK_F16) {
        a = pin_f32(a);
        b = pin_f32(b);
        uint16_t ua = __builtin_bit_cast(uint16_t, (_Float16)a);
        uint16_t ub = __builtin_bit_cast(uint16_t, (_Float16)b);
        return (uint32_t)ua | ((uint32_t)ub << 16);
    }
    uint16_t ua = __builtin_bit_cast(uint16_t, (__bf16)a);
    uint16_t ub = __builtin_bit_cast(uint16_t, (__bf16)b);
    return (uint32_t)ua | ((uint32_t)ub << 16);
}

template <int OUT_DT>
__device__ __forceinline__ void store_item(void* out, int64_t item, const float* w) {
    u32x4 v;
    if constexpr (OUT_DT == IQK_F32) {
        v.x = __float_as_uint(w[0]);
        v.y = __float_as_uint(w[1]);
        v.z = __float_as_uint(w[2]);
        v.w = __float_as_uint(w[3]);
    } else {
        v.x = pack2(w[0], w[1], OUT_DT);
        v.y = pack2(w[2], w[3], OUT_DT);
        v.z = pack2(w[4], w[5], OUT_DT);
        v.w = pack2(w[6], w[7], OUT_DT);
    }
    store16_nt(out, item, v);
}

// Raw field words of one item (the floor variant folds these into its stores).
struct ItemFields {
    uint32_t q;      // codes (2-bit members) or low index byte (IQ1_S_R4)
    uint32_t s0;     // scale word
    uint32_t s1;     // second scale / alphabet word
    uint32_t s2;     // alphabet word
    uint16_t d;      // fp16 scale
};

template <int FMT, int W>
__device__ __forceinline__ ItemFields load_item(const uint8_t* __restrict__ S, const Planes& pl, int64_t R, int64_t n,
                                                int64_t row, int64_t k0) {
    ItemFields f;
    if constexpr (FMT == IQK_IQ2_KS) {
        const int64_t sb = k0 / 32;
        const uint8_t* qs = S + pl.off[0] + row * (n / 4) + k0 / 4;
        f.q = W == 8 ? (uint32_t)*(const uint16_t*)qs : (uint32_t)*qs;
        f.s0 = S[pl.off[1] + row * (n / 64) + sb / 2];
        f.s1 = S[pl.off[2] + row * (n / 256) + sb / 8];
        f.s2 = S[pl.off[3] + row * (n / 256) + sb / 8];
        f.d = *(const uint16_t*)(S + pl.off[4] + 2 * row);
    } else if constexpr (FMT == IQK_IQ2_K) {
        const int64_t sb = k0 / 16;
        const uint8_t* qs = S + pl.off[0] + row * (n / 4) + k0 / 4;
        f.q = W == 8 ? (uint32_t)*(const uint16_t*)qs : (uint32_t)*qs;
        f.s0 = S[pl.off[1] + row * (n / 32) + sb / 2];
        f.s1 = 0;
        f.s2 = S[pl.off[2] + row * (n / 128) + sb / 8];
        f.d = *(const uint16_t*)(S + pl.off[3] + 2 * (row * (n / 256) + k0 / 256));
    } else {
        f.q = S[pl.off[0] + row * (n / 8) + k0 / 8];
        f.s0 = *(const uint16_t*)(S + pl.off[1] + 2 * (row * (n / 32) + k0 / 32));
        f.s1 = 0;
        f.s2 = 0;
        f.d = *(const uint16_t*)(S + pl.off[2] + 2 * row);
    }
    (void)R;
    return f;
}

struct DequantParams {
    const uint8_t* streams;
    Planes pl;
    int64_t R, n, row0, nrows;
    int64_t ipr;                  // items per row
    int64_t step_row, step_col;   // grid stride split as rows * ipr + cols
    float values[8];
    const int8_t* grid;
    void* out;
};

template <int FMT, int OUT_DT, bool FLOOR>
__global__ __launch_bounds__(kThreads) void dequant_kernel(DequantParams p) {
    constexpr int W = ItemShape<OUT_DT>::W;
    __shared__ float tab[8];
    if (threadIdx.x < 8) tab[threadIdx.x] = p.values[threadIdx.x];
    __syncthreads();

    const int64_t ipr = p.ipr;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    int64_t it = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    // (lr, col) walk the items without a per-item division
    int64_t lr = it / ipr;
    int64_t col = it - lr * ipr;
    for (; lr < p.nrows; it += stride, lr += p.step_row, col += p.step_col) {
        if (col >= ipr) {
            col -= ipr;
            lr += 1;
            if (lr >= p.nrows) break;
        }
        const int64_t k0 = col * W;
        const int64_t row = p.row0 + lr;
        ItemFields f = load_item<FMT, W>(p.streams, p.pl, p.R, p.n, row, k0);
        float w[W];
        if constexpr (FLOOR) {
            // deleted decode: the loaded words reach the stores unchanged
            const uint32_t h = f.q ^ (f.s0 << 8) ^ (f.s1 << 16) ^ (f.s2 << 24) ^ ((uint32_t)f.d << 5);
#pragma unroll
            for (int i = 0; i < W; ++i) w[i] = __uint_as_float(h + (uint32_t)i);
            if constexpr (OUT_DT != IQK_F32) {
                u32x4 v = {h, h ^ 1u, h ^ 2u, h ^ 3u};
                store16_nt(p.out, it, v);
                continue;
            }
        } else if constexpr (FMT == IQK_IQ2_KS) {
            const int sb = (int)((k0 / 32) & 7);
            const uint32_t lo = (f.s0 >> (4 * (sb & 1))) & 15u;
            const uint32_t hi = (f.s1 >> sb) & 1u;
            const int si = (int)(lo | (hi << 4)) - 16;
            const uint32_t alph = (f.s2 >> sb) & 1u;
            const float dl = half_bits_to_float(f.d) * (float)si;
#pragma unroll
            for (int i = 0; i < W; ++i) w[i] = dl * tab[4 * alph + ((f.q >> (2 * i)) & 3u)];
        } else if constexpr (FMT == IQK_IQ2_K) {
            const int sb = (int)((k0 / 16) & 7);
            const int si = (int)((f.s0 >> (4 * (sb & 1))) & 15u) - 8;
            const uint32_t alph = (f.s2 >> sb) & 1u;
            const float dl = half_bits_to_float(f.d) * (float)si;
#pragma unroll
            for (int i = 0; i < W; ++i) w[i] = dl * tab[4 * alph + ((f.q >> (2 * i)) & 3u)];
        } else {
            const int j = (int)((k0 / 8) & 3);
            const uint32_t idx = f.q | (((f.s0 >> (3 * j)) & 7u) << 8);
            const uint32_t ls = (f.s0 >> 12) & 7u;
            const float shift = (f.s0 >> 15) ? -0.125f : 0.125f;
            const float scale = half_bits_to_float(f.d) * (float)(2 * ls + 1);
            const int8_t* g = p.grid + 8 * idx + (k0 & 7);
            if constexpr (W == 8) {
                const uint2 gv = *(const uint2*)g;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = scale * ((float)(int8_t)(gv.x >> (8 * i)) + shift);
#pragma unroll
                for (int i = 0; i < 4; ++i) w[4 + i] = scale * ((float)(int8_t)(gv.y >> (8 * i)) + shift);
            } else {
                const uint32_t gv = *(const uint32_t*)g;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = scale * ((float)(int8_t)(gv >> (8 * i)) + shift);
            }
        }
        store_item<OUT_DT>(p.out, it, w);
    }
}

// ---------------------------------------------------------------------------
// Wide producer (in % 64 == 0): one lane decodes a 64-weight chunk of a row
// from one 16-byte code load (8 bytes for IQ1_S_R4) and three small field
// loads, stages its output in LDS, and each wave then stores its 64 chunks
// (8 or 16 KiB, contiguous in the output) as 1 KiB coalesced runs.  Cuts the
// vector-memory instructions per output byte about eightfold against one
// item per lane.
// ---------------------------------------------------------------------------

constexpr int kWideChunk = 64;  // weights per lane

template <int OUT_DT>
struct WideShape {
    static constexpr int ESZ = OUT_DT == IQK_F32 ? 4 : 2;
    static constexpr int CB = kWideChunk * ESZ;       // output bytes per lane
    static constexpr int SLOTS = CB / 16;              // 16-byte slots per lane
    static constexpr int WORDS = CB / 4;
};

// Byte offset of 16-byte slot i of lane `lane`'s run in the stage: the runs
// sit back to back (no padding) and each lane's slots are rotated by an XOR
// with its lane index, so eight lanes writing the same slot, and eight lanes
// reading one run, touch distinct banks.
template <int OUT_DT>
__device__ __forceinline__ int stage_off(int lane, int i) {
    using WS = WideShape<OUT_DT>;
    return lane * WS::CB + 16 * (i ^ (lane & (WS::SLOTS - 1)));
}

template <int OUT_DT>
__device__ __forceinline__ uint32_t cvt_pair(float a, float b) {
    if constexpr (OUT_DT == IQK_F16) {
        a = pin_f32(a);
        b = pin_f32(b);
        return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16);
    } else {
        return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a) | ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)b) << 16);
    }
}

// The stream words of one 64-weight chunk (codes and the per-chunk fields;
// unused members zero).
struct ChunkWords {
    uint4 q;
    uint32_t a, b, c, d;
};

template <int FMT>
__device__ __forceinline__ ChunkWords load_chunk(const DequantParams& p, int64_t row, int64_t c) {
    const uint8_t* S = p.streams;
    const int64_t n = p.n;
    ChunkWords w{};
    if constexpr (FMT == IQK_IQ2_KS) {
        w.q = *(const uint4*)(S + p.pl.off[0] + row * (n / 4) + 16 * c);
        w.a = S[p.pl.off[1] + row * (n / 64) + c];
        w.b = S[p.pl.off[2] + row * (n / 256) + c / 4];
        w.c = S[p.pl.off[3] + row * (n / 256) + c / 4];
        w.d = *(const uint16_t*)(S + p.pl.off[4] + 2 * row);
    } else if constexpr (FMT == IQK_IQ2_K) {
        w.q = *(const uint4*)(S + p.pl.off[0] + row * (n / 4) + 16 * c);
        w.a = *(const uint16_t*)(S + p.pl.off[1] + row * (n / 32) + 2 * c);
        w.b = S[p.pl.off[2] + row * (n / 128) + c / 2];
        w.d = *(const uint16_t*)(S + p.pl.off[3] + row * (n / 128) + 2 * (c / 4));
    } else {
        const uint2 q = *(const uint2*)(S + p.pl.off[0] + row * (n / 8) + 8 * c);
        w.q = make_uint4(q.x, q.y, 0u, 0u);
        w.a = *(const uint32_t*)(S + p.pl.off[1] + row * (n / 16) + 4 * c);
        w.d = *(const uint16_t*)(S + p.pl.off[2] + 2 * row);
    }
    return w;
}

// Decode one 64-weight chunk (column c; its words already loaded) into
// output words (f32: 64 words, f16/bf16: 32).
template <int FMT, int OUT_DT, bool FLOOR>
__device__ __forceinline__ void decode_chunk(const DequantParams& p, const ChunkWords& cw, int64_t c,
                                             const float* tab, const uint2* grid_s, const uint16_t* grid_p,
                                             uint32_t* o) {
    float w[kWideChunk];
    if constexpr (FMT == IQK_IQ2_KS) {
        const uint4 q = cw.q;
        const uint32_t scl = cw.a;
        const uint32_t sch = cw.b;
        const uint32_t sex = cw.c;
        const uint32_t d = cw.d;
        if constexpr (FLOOR) {
            const uint32_t h = q.x ^ q.y ^ q.z ^ q.w ^ (scl << 8) ^ (sch << 16) ^ (sex << 24) ^ (d << 3);
#pragma unroll
            for (int i = 0; i < WideShape<OUT_DT>::WORDS; ++i) o[i] = h + (uint32_t)i;
            return;
        } else {
            const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
            const int sh = 2 * (int)(c & 3);
#pragma unroll
            for (int sbl = 0; sbl < 2; ++sbl) {
                const int si = (int)(((scl >> (4 * sbl)) & 15u) | (((sch >> (sh + sbl)) & 1u) << 4)) - 16;
                const uint32_t alph = (sex >> (sh + sbl)) & 1u;
                const float dl = half_bits_to_float((uint16_t)d) * (float)si;
#pragma unroll
                for (int i = 0; i < 32; ++i)
                    w[32 * sbl + i] = dl * tab[4 * alph + ((qw[2 * sbl + (i >> 4)] >> (2 * (i & 15))) & 3u)];
            }
        }
    } else if constexpr (FMT == IQK_IQ2_K) {
        const uint4 q = cw.q;
        const uint32_t scl = cw.a;
        const uint32_t sex = cw.b >> (4 * (c & 1));
        const uint32_t d = cw.d;
        if constexpr (FLOOR) {
            const uint32_t h = q.x ^ q.y ^ q.z ^ q.w ^ (scl << 8) ^ (sex << 24) ^ (d << 3);
#pragma unroll
            for (int i = 0; i < WideShape<OUT_DT>::WORDS; ++i) o[i] = h + (uint32_t)i;
            return;
        } else {
            const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
            const float df = half_bits_to_float((uint16_t)d);
#pragma unroll
            for (int sbl = 0; sbl < 4; ++sbl) {
                const int si = (int)((scl >> (4 * sbl)) & 15u) - 8;
                const uint32_t alph = (sex >> sbl) & 1u;
                const float dl = df * (float)si;
#pragma unroll
                for (int i = 0; i < 16; ++i) w[16 * sbl + i] = dl * tab[4 * alph + ((qw[sbl] >> (2 * i)) & 3u)];
            }
        }
    } else {
        const uint2 q = make_uint2(cw.q.x, cw.q.y);
        const uint32_t qh = cw.a;
        const uint32_t d = cw.d;
        if constexpr (FLOOR) {
            const uint32_t h = q.x ^ q.y ^ qh ^ (d << 3);
#pragma unroll
            for (int i = 0; i < WideShape<OUT_DT>::WORDS; ++i) o[i] = h + (uint32_t)i;
            return;
        } else if constexpr (OUT_DT != IQK_F32) {
            // A 32-weight block takes three values, scale * (g + shift) for
            // g = 0, +1, -1, each rounded once to the output type: a 4-entry
            // table indexed by the grid byte & 3 (0, 1, 3), split into low and
            // high bytes so one v_perm_b32 builds a weight pair from a
            // selector that one more v_perm_b32 makes from the grid bytes.
            const float df = half_bits_to_float((uint16_t)d);
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const uint32_t h16 = (qh >> (16 * b)) & 0xFFFFu;
                const float scale = df * (float)(2 * ((h16 >> 12) & 7u) + 1);
                const float shift = (h16 >> 15) ? -0.125f : 0.125f;
                const uint32_t p0 = cvt_pair<OUT_DT>(scale * (0.0f + shift), scale * (1.0f + shift));
                const uint32_t p1 = cvt_pair<OUT_DT>(0.0f, scale * (-1.0f + shift));
                const uint32_t tlo = __builtin_amdgcn_perm(p1, p0, 0x06040200u);
                const uint32_t thi = __builtin_amdgcn_perm(p1, p0, 0x07050301u);
                const uint32_t qsw = b == 0 ? q.x : q.y;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t idx = ((qsw >> (8 * j)) & 0xFFu) | (((h16 >> (3 * j)) & 7u) << 8);
                    // the packed entry: nibble k holds the codes of values k
                    // and k + 4; one v_perm_b32 spreads the nibbles to bytes
                    const uint32_t e = grid_p[idx];
                    const uint32_t wv = __builtin_amdgcn_perm(e >> 4, e, 0x05010400u);
                    const uint32_t vx = wv & 0x03030303u, vy = (wv >> 2) & 0x03030303u;
                    const uint32_t vx4 = vx | 0x04040404u, vy4 = vy | 0x04040404u;
                    // selectors [c_a, 4 + c_a, c_b, 4 + c_b] for the pairs (0, 1) and (2, 3)
                    o[16 * b + 4 * j + 0] = __builtin_amdgcn_perm(thi, tlo, __builtin_amdgcn_perm(vx4, vx, 0x05010400u));
                    o[16 * b + 4 * j + 1] = __builtin_amdgcn_perm(thi, tlo, __builtin_amdgcn_perm(vx4, vx, 0x07030602u));
                    o[16 * b + 4 * j + 2] = __builtin_amdgcn_perm(thi, tlo, __builtin_amdgcn_perm(vy4, vy, 0x05010400u));
                    o[16 * b + 4 * j + 3] = __builtin_amdgcn_perm(thi, tlo, __builtin_amdgcn_perm(vy4, vy, 0x07030602u));
                }
            }
            return;
        } else {
            const float df = half_bits_to_float((uint16_t)d);
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const uint32_t h16 = (qh >> (16 * b)) & 0xFFFFu;
                const float scale = df * (float)(2 * ((h16 >> 12) & 7u) + 1);
                const float shift = (h16 >> 15) ? -0.125f : 0.125f;
                const uint32_t qsw = b == 0 ? q.x : q.y;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t idx = ((qsw >> (8 * j)) & 0xFFu) | (((h16 >> (3 * j)) & 7u) << 8);
                    const uint2 gv = grid_s[idx];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        w[32 * b + 8 * j + i] = scale * ((float)(int8_t)(gv.x >> (8 * i)) + shift);
                        w[32 * b + 8 * j + 4 + i] = scale * ((float)(int8_t)(gv.y >> (8 * i)) + shift);
                    }
                }
            }
        }
    }
    if constexpr (!FLOOR) {
        if constexpr (OUT_DT == IQK_F32) {
#pragma unroll
            for (int i = 0; i < kWideChunk; ++i) o[i] = __float_as_uint(w[i]);
        } else {
#pragma unroll
            for (int i = 0; i < kWideChunk / 2; ++i) o[i] = cvt_pair<OUT_DT>(w[2 * i], w[2 * i + 1]);
        }
    }
}

// Low two bits of each value's byte packed into a 16-bit grid entry: nibble
// k = code(value k) | code(value k + 4) << 2, for the two words w of an
// entry (values 0-3 in w0, 4-7 in w1).
__device__ __forceinline__ uint32_t pack_codes(uint32_t w0, uint32_t w1) {
    const uint32_t nib = (w0 & 0x03030303u) | ((w1 & 0x03030303u) << 2);  // byte k: nibble k
    return (nib & 0xFu) | ((nib >> 4) & 0xF0u) | ((nib >> 8) & 0xF00u) | ((nib >> 12) & 0xF000u);
}

template <int FMT, int OUT_DT, bool FLOOR, bool AHEAD>
__global__ __launch_bounds__(kThreads) void dequant_wide_kernel(DequantParams p) {
    using WS = WideShape<OUT_DT>;
    // f16 / bf16 output of IQ1_S_R4 looks each weight up among the three
    // values a ternary grid gives, so its LDS copy of the grid keeps only
    // each value's two low bits (4 KiB: with the 32 KiB stage, four
    // workgroups fit a CU's LDS); a grid holding any other value makes the
    // whole output NaN (checked while the grid is staged).  The float32
    // output takes any int8 value and stages the whole grid.
    constexpr bool kTernary = FMT == IQK_IQ1_S_R4 && OUT_DT != IQK_F32 && !FLOOR;
    constexpr bool kWholeGrid = FMT == IQK_IQ1_S_R4 && OUT_DT == IQK_F32 && !FLOOR;
    __shared__ float tab[FMT == IQK_IQ1_S_R4 ? 1 : 8];
    __shared__ uint2 grid_s[kWholeGrid ? 2048 : 1];
    __shared__ uint16_t grid_p[kTernary ? 2048 : 1];
    __shared__ __attribute__((aligned(16))) uint8_t stage[kThreads * WS::CB];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    if constexpr (FMT != IQK_IQ1_S_R4) {
        if (tid < 8) tab[tid] = p.values[tid];
    }
    uint32_t off_grid = 0;
    if constexpr (kWholeGrid) {
        const uint4* src = (const uint4*)p.grid;
        uint4* dst = (uint4*)grid_s;
        for (int i = tid; i < 1024; i += kThreads) dst[i] = src[i];
    } else if constexpr (kTernary) {
        const uint4* src = (const uint4*)p.grid;  // two entries per 16 bytes
        for (int i = tid; i < 1024; i += kThreads) {
            const uint4 v = src[i];
            off_grid |= non_ternary(v.x) | non_ternary(v.y) | non_ternary(v.z) | non_ternary(v.w);
            *(uint32_t*)&grid_p[2 * i] = pack_codes(v.x, v.y) | (pack_codes(v.z, v.w) << 16);
        }
    }
    const bool nan_out = kTernary ? __syncthreads_or(off_grid != 0) != 0 : (__syncthreads(), false);

    const int64_t cpr = p.ipr;                 // chunks per row
    const int64_t chunks = p.nrows * cpr;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    uint8_t* wst = stage + wave * 64 * WS::CB;  // the wave's runs
    const int64_t total_bytes = chunks * WS::CB;
    int64_t ch = (int64_t)blockIdx.x * kThreads + tid;
    int64_t lr = ch / cpr;
    int64_t col = ch - lr * cpr;
    // AHEAD: each lane requests its next chunk's words before decoding the
    // current one, so their latency runs under the decode and the stores (the
    // compiler keeps loads behind earlier stores to the output, which it
    // cannot prove disjoint from the streams).  Otherwise each chunk's words
    // are loaded just before it is decoded.
    constexpr bool ahead = AHEAD;
    ChunkWords cur{};
    if (ahead && ch < chunks) cur = load_chunk<FMT>(p, p.row0 + lr, col);
    for (int64_t base = (int64_t)blockIdx.x * kThreads + wave * 64; base < chunks;
         base += stride, ch += stride, lr += p.step_row, col += p.step_col) {
        if (col >= cpr) {
            col -= cpr;
            lr += 1;
        }
        ChunkWords nxt{};
        if constexpr (ahead) {
            int64_t nlr = lr + p.step_row, ncol = col + p.step_col;
            if (ncol >= cpr) {
                ncol -= cpr;
                nlr += 1;
            }
            if (ch + stride < chunks) nxt = load_chunk<FMT>(p, p.row0 + nlr, ncol);
        } else if (ch < chunks) {
            cur = load_chunk<FMT>(p, p.row0 + lr, col);
        }
        if (ch < chunks) {
            uint32_t o[WS::WORDS];
            decode_chunk<FMT, OUT_DT, FLOOR>(p, cur, col, tab, grid_s, grid_p, o);
            if (kTernary && nan_out) {
#pragma unroll
                for (int i = 0; i < WS::WORDS; ++i) o[i] = OUT_DT == IQK_F16 ? 0x7E007E00u : 0x7FC07FC0u;
            }
#pragma unroll
            for (int i = 0; i < WS::SLOTS; ++i)
                *(uint4*)(wst + stage_off<OUT_DT>(lane, i)) = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // the wave's 64 chunks are contiguous in the output: store 1 KiB runs
        const int64_t out0 = base * WS::CB;
#pragma unroll
        for (int s2 = 0; s2 < WS::CB / 16; ++s2) {
            const int o = s2 * 1024 + 16 * lane;          // byte offset within the wave's output run
            const int src_lane = o / WS::CB, within = o % WS::CB;
            const int64_t ob = out0 + o;
            if (ob < total_bytes) {
                const uint4 v = *(const uint4*)(wst + stage_off<OUT_DT>(src_lane, within / 16));
                u32x4 vv = {v.x, v.y, v.z, v.w};
                __builtin_nontemporal_store(vv, (u32x4*)((uint8_t*)p.out + ob));
            }
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if constexpr (ahead) cur = nxt;
    }
}

template <int FMT, int OUT_DT, bool FLOOR>
hipError_t launch_wide(DequantParams p, hipStream_t s) {
    // loads one chunk ahead for IQ1_S_R4 (its grid lookups lengthen every
    // chunk's dependency chain) and for rows of at most 2048 weights.
    // Measured (bf16 out, 256 experts): IQ1_S_R4 gate/up 1800 -> 1626 us,
    // down 867 -> 793 us; IQ2_K down 858 -> 818 us, IQ2_KS down 808 -> 789
    // us; the 2-bit members' 4096-wide rows were 1-6 % slower ahead.
    const bool ahead = FMT == IQK_IQ1_S_R4 || p.n <= 2048;
    p.ipr = p.n / kWideChunk;
    const int64_t chunks = p.nrows * p.ipr;
    constexpr int64_t kPerThread = FMT == IQK_IQ1_S_R4 && !FLOOR ? IQK_DEQUANT_GRID_CHUNKS : 1;
    // IQ2_K: one chunk per lane up to twice the usual cap (its 4096-wide
    // gate/up rows 1712 -> 1622 us with one pass instead of two; IQ2_KS
    // measured 3 % slower that way, IQ1_S_R4 unchanged)
    const int64_t cap = FMT == IQK_IQ2_K ? 2 * (int64_t)IQK_DEQUANT_MAX_BLOCKS : (int64_t)IQK_DEQUANT_MAX_BLOCKS;
    int64_t blocks = (chunks + kPerThread * kThreads - 1) / (kPerThread * kThreads);
    blocks = blocks < cap ? blocks : cap;
    if (blocks < 1) blocks = 1;
    const int64_t stride = blocks * kThreads;
    p.step_row = stride / p.ipr;
    p.step_col = stride % p.ipr;
    if (ahead)
        hipLaunchKernelGGL((dequant_wide_kernel<FMT, OUT_DT, FLOOR, true>), dim3((unsigned)blocks), dim3(kThreads), 0,
                           s, p);
    else
        hipLaunchKernelGGL((dequant_wide_kernel<FMT, OUT_DT, FLOOR, false>), dim3((unsigned)blocks), dim3(kThreads), 0,
                           s, p);
    return hipGetLastError();
}

template <int FMT, int OUT_DT, bool FLOOR>
hipError_t launch_one(DequantParams p, hipStream_t s) {
    if (p.n % kWideChunk == 0) return launch_wide<FMT, OUT_DT, FLOOR>(p, s);
    constexpr int W = ItemShape<OUT_DT>::W;
    p.ipr = p.n / W;
    const int64_t items = p.nrows * p.ipr;
    int64_t blocks = (items + kThreads - 1) / kThreads;
    // enough workgroups to fill 256 CUs many times over; the grid strides
    blocks = blocks < IQK_DEQUANT_MAX_BLOCKS ? blocks : IQK_DEQUANT_MAX_BLOCKS;
    if (blocks < 1) blocks = 1;
    const int64_t stride = blocks * kThreads;
    p.step_row = stride / p.ipr;
    p.step_col = stride % p.ipr;
    hipLaunchKernelGGL((dequant_kernel<FMT, OUT_DT, FLOOR>), dim3((unsigned)blocks), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <int FMT, bool FLOOR>
hipError_t launch_fmt(const DequantParams& p, int out_dt, hipStream_t s) {
    if (out_dt == IQK_F32) return launch_one<FMT, IQK_F32, FLOOR>(p, s);
    if (out_dt == IQK_F16) return launch_one<FMT, IQK_F16, FLOOR>(p, s);
    return launch_one<FMT, IQK_BF16, FLOOR>(p, s);
}

template <bool FLOOR>
hipError_t launch_any(const DequantParams& p, int fmt, int out_dt, hipStream_t s) {
    if (fmt == IQK_IQ2_KS) return launch_fmt<IQK_IQ2_KS, FLOOR>(p, out_dt, s);
    if (fmt == IQK_IQ2_K) return launch_fmt<IQK_IQ2_K, FLOOR>(p, out_dt, s);
    return launch_fmt<IQK_IQ1_S_R4, FLOOR>(p, out_dt, s);
}

}  // namespace

hipError_t launch_dequant(const DequantLaunch& a, bool floor_variant, hipStream_t s) {
    DequantParams p;
    p.streams = a.streams;
    p.pl = a.pl;
    p.R = a.R;
    p.n = a.n;
    p.row0 = a.row0;
    p.nrows = a.nrows;
    for (int i = 0; i < 8; ++i) p.values[i] = a.values[i];
    p.grid = a.grid;
    p.out = a.out;
    return floor_variant ? launch_any<true>(p, a.fmt, a.out_dtype, s) : launch_any<false>(p, a.fmt, a.out_dtype, s);
}

}  // namespace iqk
