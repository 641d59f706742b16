/*
 * iqk.h -- C ABI of the MI355X (gfx950) IQ_K routed-expert library.
 *
 * The operations follow the "mlx-iqk" package description (IQ_K relayout
 * routed-expert kernels):
 *   - "Format" section: the per-row streams of IQ2_KS (qs, scl, sch, sex,
 *     dv), IQ2_K (qs, scl, sex, dv) and IQ1_S_R4 (qs, qh, dv); the two float32
 *     reconstruction chains; the row budgets 2 + 70n/256, 76n/256 and
 *     2 + 6n/32 bytes; the IQ1_S_R4 wire in whole four-row groups;
 *   - introduction: the build-time relayout that makes values consumed
 *     along k contiguous without changing a value or a byte budget;
 *   - "Surface" section: the switch-linear call y = proj(x, indices): few
 *     token-expert pairs run a fused decode matvec, many pairs run a
 *     one-pass dequantization of the stacked experts followed by a grouped
 *     GEMM that reads each expert once when pairs are sorted by expert; the
 *     decode kernel exists only for instantiated input widths and any other
 *     width is refused.
 *
 * Conventions for every call:
 *   - Plain pointers and sizes.  "host" pointers are CPU memory, "device"
 *     pointers are HIP device memory of the current device.  The caller owns
 *     every buffer; the library allocates nothing and keeps no state except a
 *     per-thread error message.
 *   - Every argument is validated before any HIP call.  A failed check
 *     returns a negative iqk_status, touches no buffer, enqueues nothing and
 *     sets iqk_last_error().
 *   - Device calls enqueue on `stream` (a hipStream_t; NULL = the null
 *     stream) and return without synchronizing.  Launch failures return
 *     IQK_E_HIP with the HIP error text in iqk_last_error().
 *   - Calls that overlap on one stream are ordered; calls on different
 *     streams that write the same output race.
 *
 * Stream tensors ("served relayout", canonical layout of this library).  A
 * weight descriptor covers E experts of [out, in] stacked to R = E*out rows.
 * Each stream is a plane over all R rows, row-major, k-contiguous, with no
 * padding; planes follow the order of the stream tables; bits are LSB-first
 * within bytes (equivalently, element i of a plane of w-bit elements sits at
 * bits [w*i mod 32, +w) of little-endian uint32 word w*i/32):
 *   IQ2_KS  (in % 256 == 0): qs R*in/4 (2-bit code per weight) | scl R*in/64
 *           (4-bit low part of the scale index per 32 weights) | sch R*in/256
 *           (high bit per 32 weights) | sex R*in/256 (alphabet bit per 32
 *           weights) | dv R*2 (fp16 row scale).
 *           scale_index = (scl | sch << 4) - 16, in [-16, 15].
 *   IQ2_K   (in % 256 == 0): qs R*in/4 | scl R*in/32 (4-bit per 16 weights,
 *           scale_index = scl - 8) | sex R*in/128 (bit per 16 weights) |
 *           dv R*(in/256)*2 (fp16 per 256 weights).
 *   IQ1_S_R4 (in % 32 == 0): qs R*in/8 (low 8 bits of the 11-bit grid index
 *           per 8 weights; block b of 32 weights is uint32 word b) |
 *           qh R*(in/32)*2 (uint16 per 32 weights: bits 3j..3j+2 = index high
 *           bits of group j, bits 12..14 = ls, bit 15 = shift sign, set means
 *           -0.125) | dv R*2 (fp16 row scale).
 * Reconstruction (float32, every step rounded, in this order):
 *   2-bit:   w = (float(dv) * float(scale_index)) * values[4*alphabet + code]
 *   IQ1_S_R4: w = (float(dv) * float(2*ls + 1)) * (float(grid[idx][k%8]) + shift)
 *
 * Wire tensors (ik block structs, per "Format": the same byte budgets).
 * The bit positions inside the blocks are this library's stand-in reading:
 *   IQ2_KS per row: fp16 d, then in/256 blocks of 70 B {uint16 extra (bit s =
 *     alphabet of sub-block s, bit 8+s = scale high bit), uint8 scales[4]
 *     (low nibble sub-block 2i, high nibble 2i+1), uint8 qs[64]}.
 *   IQ2_K per row: in/256 blocks of 76 B {fp16 d, uint16 extra (bit s =
 *     alphabet of sub-block s), uint8 scales[8], uint8 qs[64]}.
 *   qs of both: weight 128h + 32p + l of a block -> byte 32h + l, bits 2p.
 *   IQ1_S_R4 per four-row group: fp16 d[4], then in/32 blocks of 24 B
 *     {uint8 qs[16] (byte 4j + r = group j of row r), uint16 qh[4]}.
 */
#ifndef IQK_H
#define IQK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { IQK_IQ2_KS = 1, IQK_IQ2_K = 2, IQK_IQ1_S_R4 = 3 } iqk_format;
typedef enum { IQK_F32 = 0, IQK_F16 = 1, IQK_BF16 = 2 } iqk_dtype;
typedef enum {
    IQK_OK = 0,
    IQK_E_ARG = -1,     /* null pointer, negative size, bad enum, bad count */
    IQK_E_FORMAT = -2,  /* unknown format */
    IQK_E_SHAPE = -3,   /* in % 256 (2-bit members) or in % 32 (IQ1_S_R4) != 0 */
    IQK_E_WIDTH = -4,   /* decode matvec: no instance for this input width */
    IQK_E_ROWS4 = -5,   /* IQ1_S_R4 wire: rows not a multiple of four */
    IQK_E_SIZE = -6,    /* a byte count does not match the layout */
    IQK_E_TABLE = -7,   /* decode matvec: value table not of the form m_i * 2^e, |m_i| <= 127 */
    IQK_E_HIP = -8      /* HIP runtime error */
} iqk_status;

/* Expert-stacked weights: `experts` tensors of [out, in], R = experts*out rows
 * in the canonical stream layout above.  `streams` is a device pointer of
 * exactly `streams_bytes` = R * iqk_row_bytes(fmt, in) bytes. */
typedef struct iqk_weights {
    int32_t fmt;
    int64_t experts, out, in;
    const void* streams;
    size_t streams_bytes;
} iqk_weights;

/* Bytes of one row of `n` weights ("Format": row budgets); 0 if the format is
 * unknown or n violates its shape rule. */
size_t iqk_row_bytes(int fmt, int64_t n);

/* Byte offsets of the planes of an R-row stream tensor (unused entries = -1):
 * IQ2_KS {qs, scl, sch, sex, dv}; IQ2_K {qs, scl, sex, dv, -1};
 * IQ1_S_R4 {qs, qh, dv, -1, -1}.  *total = R * iqk_row_bytes(fmt, n). */
int iqk_plane_offsets(int fmt, int64_t rows, int64_t n, int64_t off[5], int64_t* total);

/* Relayout ("Format" / introduction): wire -> canonical streams, a pure bit
 * permutation with equal byte counts.  Host memory, synchronous.  Both
 * buffers must hold exactly rows * iqk_row_bytes(fmt, n) bytes; IQ1_S_R4
 * needs rows % 4 == 0 (IQK_E_ROWS4).  `wire` and `streams` must not overlap. */
int iqk_pack_relayout(int fmt, const uint8_t* wire, size_t wire_bytes, int64_t rows, int64_t n,
                      uint8_t* streams, size_t streams_bytes);
/* The inverse permutation: canonical streams -> wire. */
int iqk_unpack_relayout(int fmt, const uint8_t* streams, size_t streams_bytes, int64_t rows, int64_t n,
                        uint8_t* wire, size_t wire_bytes);

/* Dequantization ("Format" reconstruction; the prefill weight producer of
 * "Surface"): rows [row0, row0 + nrows) of the stacked tensor -> `out`
 * [nrows, in] (device, dense, row-major) in `out_dtype`.  float32 results
 * are bit-exact with the float32 chain; f16 / bf16 results are one
 * round-to-nearest-even cast of it (NaN results are quiet NaNs of
 * unspecified payload).
 * `values`: host float[8] for the 2-bit members (any float32 values),
 * ignored for IQ1_S_R4.  `grid`: device int8[2048*8] (row idx = 8 grid
 * values) for IQ1_S_R4, ignored otherwise.  Precondition of the f16 / bf16
 * output when in % 64 == 0: the grid is ternary (-1, 0, +1, the grid's
 * definition), since each weight is looked up among the three rounded
 * values its block can take; the kernel checks the grid as it loads it and
 * writes NaN to every output if any value is outside {-1, 0, +1}.  The
 * float32 output (and f16 / bf16 at other widths) computes any int8 grid
 * value. */
int iqk_dequant(const iqk_weights* w, int64_t row0, int64_t nrows, const float* values,
                const int8_t* grid, int out_dtype, void* out, void* stream);

/* Fused decode matvec ("Surface": few token-expert pairs).
 * y[t, j, o] = sum_k W_{ids[t,j]}[o, k] * x[t, s, k] with s = 0 if
 * x_slots == 1 (shared input, gate/up) or s = j if x_slots == k (per-pair
 * input, down).  x: device [T, x_slots, in] of x_dtype IQK_F32 or IQK_BF16,
 * finite (a NaN or infinite activation gives an unspecified result).
 * ids: device int32 [T, k]; an id outside [0, experts) gives a NaN output
 * row (the rule of every routed-product call of this library).
 * y: device float32 [T, k, out].
 * Widths: in must be 512, 2048 or 4096 (IQK_E_WIDTH otherwise): a kernel
 * instance makes exactly one pass over k.  The values table (host float[8])
 * must be m_i * 2^e with integer |m_i| <= 127 for one common e (integer
 * tables qualify), else IQK_E_TABLE.  Accuracy: the activation is held per
 * 64-value block as 15-bit fixed point (relative error about 2^-14 of the
 * block maximum); weights and sums are exact integers up to one float32
 * rounding per row; ||y - y_exact|| / ||y_exact|| <= 1e-3.
 * Limits: T * k <= 65535 * 64, out * iqk_row_bytes(fmt, in) < 2^31,
 * T * k * ceil(out / 4) < 2^31 (IQK_E_ARG otherwise). */
int iqk_moe_gemv(const iqk_weights* w, const float* values, const int8_t* grid,
                 const void* x, int x_dtype, int x_slots, const int32_t* ids,
                 int64_t T, int k, float* y, void* stream);

/* The MoE layer step after gate/up (the projection-level interface of
 * "Surface" used the way a SwiGLU expert uses it): the same matvec over a
 * gate/up tensor whose rows [0, I) are gate and [I, 2I) up (out = 2I, even,
 * else IQK_E_SHAPE), written as h[t, j, i] = silu(g) * u with
 * g = gate_i . x, u = up_i . x, silu(g) = g / (1 + exp(-g)) in float32 (the
 * hardware exponential and reciprocal, about an ulp each), and h stored as
 * bf16 (round to nearest even): device uint16 [T, k, I].  This is
 * the down projection's per-pair input.  Invalid ids give NaN rows.
 * Arguments and limits otherwise as iqk_moe_gemv. */
int iqk_moe_gemv_swiglu(const iqk_weights* w, const float* values, const int8_t* grid,
                        const void* x, int x_dtype, int x_slots, const int32_t* ids,
                        int64_t T, int k, uint16_t* h, void* stream);

/* The MoE layer step after down: router-weighted combine of the k routed
 * experts, y[t, o] = sum_{j=0..k-1} route_w[t, j] * (W_{ids[t,j]}[o, :] .
 * x[t, s, :]), summed in float32 in slot order (s as in iqk_moe_gemv).
 * route_w: device float32 [T, k]; y: device float32 [T, out].  An invalid
 * id makes its token's row NaN.  k <= 8 (IQK_E_ARG); otherwise as
 * iqk_moe_gemv.  Deterministic: one wave owns each (token, row group). */
int iqk_moe_gemv_combine(const iqk_weights* w, const float* values, const int8_t* grid,
                         const void* x, int x_dtype, int x_slots, const int32_t* ids,
                         const float* route_w, int64_t T, int k, float* y, void* stream);

/* Workspace of iqk_moe_gemv_grouped: the routing arrays (counts, offsets,
 * permutation) and a work plan of E + 1 int64, each rounded up to 256
 * bytes. */
int iqk_moe_gemv_grouped_workspace(const iqk_weights* w, int64_t T, int k, size_t* bytes);

/* Grouped decode matvec for a few tokens per expert (between the per-pair
 * matvec and the prefill in "Surface"'s dispatch by the number of
 * token-expert pairs): iqk_route, then one pass over each selected expert's
 * rows that decodes every 64-weight chunk once and multiplies it with all of
 * the expert's pairs (4 per pass for a bf16 activation, 3 for float32; the
 * pass's activations are held in registers), so an expert chosen by several
 * tokens is read and decoded once per pass.  Arguments, value-table rule, accuracy
 * and widths as iqk_moe_gemv; workspace from iqk_moe_gemv_grouped_workspace;
 * `sorted` as iqk_route.  Per pair the sums are formed as in iqk_moe_gemv
 * (the two agree to float32 rounding).  Pairs with an invalid id get NaN
 * rows, as in iqk_moe_gemv (the routing drops them and writes those rows).
 * Limits: as iqk_moe_gemv, E <= 16384, T * k * out * 4 < 2^31. */
int iqk_moe_gemv_grouped(const iqk_weights* w, const float* values, const int8_t* grid,
                         const void* x, int x_dtype, int x_slots, const int32_t* ids,
                         int64_t T, int k, int sorted, void* workspace, size_t ws_bytes,
                         float* y, void* stream);

/* Workspace of iqk_moe_auto (that of iqk_moe_gemv_grouped, which equals
 * that of iqk_moe_prefill_fused). */
int iqk_moe_auto_workspace(const iqk_weights* w, int64_t T, int k, size_t* bytes);

/* The routed projection y[T, k, out] with the path chosen by the number of
 * token-expert pairs ("Surface": few pairs take the fused decode, many the
 * prefill), with the crossover measured on the routed geometry (top-6 of
 * 256 experts): pairs per expert T*k/E <= 3/4 -> iqk_moe_gemv; above
 * that, for in = 4096, <= 3/2 -> iqk_moe_gemv_grouped and above ->
 * iqk_moe_prefill_fused; for narrower inputs iqk_moe_prefill_fused.  A float32 activation never takes the prefill
 * (it needs bf16); a value table that is not int8-exact takes the prefill
 * when x is bf16 (else IQK_E_TABLE).  *path (if non-null) receives 0, 1 or
 * 2 for the path taken.  Arguments and errors are those of the chosen call;
 * accuracy is that call's (1e-3 for the matvecs, 2e-2 for the prefill).  Rows
 * of pairs with an invalid id are NaN on every path. */
int iqk_moe_auto(const iqk_weights* w, const float* values, const int8_t* grid,
                 const void* x, int x_dtype, int x_slots, const int32_t* ids, int64_t T, int k,
                 void* workspace, size_t ws_bytes, float* y, int* path, void* stream);

/* iqk_moe_auto for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, hosts that forbid allocation): no
 * workspace argument; the routing arrays and the work plan live in a fixed
 * device array of the library (1 MiB on each GPU it runs on, held until
 * the process ends; its address is taken once per device, on the first
 * call with that device current).  A call whose
 * iqk_moe_auto_workspace exceeds 1 MiB returns IQK_E_SIZE (at 256 experts
 * about 260 k token-expert pairs fit).  The call allocates nothing.  Every
 * call on one GPU shares that GPU's array and rebuilds its contents, so
 * calls that overlap on one GPU (different streams, or threads) race.
 * Arguments, results and errors otherwise as iqk_moe_auto. */
int iqk_moe_auto_noalloc(const iqk_weights* w, const float* values, const int8_t* grid,
                         const void* x, int x_dtype, int x_slots, const int32_t* ids, int64_t T, int k,
                         float* y, int* path, void* stream);

/* The layer steps either side of the projections for the prefill paths
 * (the decode matvec has them as epilogues: iqk_moe_gemv_swiglu,
 * iqk_moe_gemv_combine), with the same arithmetic (SwiGLU of the same
 * gate/up sums gives the same bits; the combine agrees to float32
 * rounding).  iqk_swiglu: y_gu device float32 [P, 2I] (per pair, gate
 * columns [0, I) then up columns [I, 2I), as a gate/up projection writes
 * them) -> h device bf16 [P, I], h = silu(g) * u as in
 * iqk_moe_gemv_swiglu, one round-to-nearest-even cast.  I % 4 == 0
 * (IQK_E_SHAPE); y_gu 16-byte and h 8-byte aligned.  iqk_combine: y device
 * float32 [T, k, out], route_w device float32 [T, k] -> yc device float32
 * [T, out], yc[t] = sum_j route_w[t, j] * y[t, j] (each product rounded,
 * summed in slot order j = 0..k-1; a NaN in a slot makes that output NaN).
 * out % 4 == 0 (IQK_E_SHAPE); y and yc 16-byte aligned. */
int iqk_swiglu(const float* y_gu, int64_t P, int64_t I, uint16_t* h, void* stream);
int iqk_combine(const float* y, const float* route_w, int64_t T, int k, int64_t out, float* yc,
                void* stream);

/* Routing gather ("Surface": sorting pairs by expert so that each expert's
 * weights are read once).  ids: device int32 [P] (P = T*k pair indices
 * t*k + j).  Writes device int32 counts[E], offsets[E+1] (exclusive prefix
 * sum) and perm[P]: pair indices grouped by increasing expert, increasing
 * pair index inside an expert (a stable sort); pairs with an id outside
 * [0, E) are dropped and the remaining perm entries are set to -1.
 * `sorted` = 1 is the caller's sort flag ("Surface"): it states that ids
 * are non-decreasing, in which case the stable sort is the identity on the
 * valid pairs and the kernel skips the ranking.  The kernel confirms the
 * order while it counts (ids not in order take the full ranking), so the
 * result is the same either way.  P <= 2^24, E <= 16384. */
int iqk_route(const int32_t* ids, int64_t P, int64_t E, int sorted,
              int32_t* counts, int32_t* offsets, int32_t* perm, void* stream);

/* Grouped GEMM over expert-stacked dense bf16 weights (MLX's gather_mm in
 * "Surface"): for every routed pair p = t*k + j with expert e,
 * y[p, :] = W[e] @ x[t, s, :] (s as in iqk_moe_gemv), bf16 inputs, float32
 * accumulation on MFMA.  W: device bf16 [E, out, in]; x: device bf16
 * [T, x_slots, in]; offsets / perm from iqk_route; y: device float32
 * [T, k, out]; rows of dropped pairs are left untouched.  in % 64 == 0,
 * out % 16 == 0, E <= 16384. */
int iqk_grouped_gemm(const void* W_bf16, int64_t E, int64_t out, int64_t in,
                     const void* x_bf16, int x_slots, int64_t T, int k,
                     const int32_t* offsets, const int32_t* perm, float* y, void* stream);

/* Workspace of iqk_moe_prefill_fused: the routing arrays (counts, offsets,
 * permutation) and a work plan of E + 1 int64 (each expert's share of the
 * kernel's work), each rounded up to 256 bytes. */
int iqk_moe_prefill_fused_workspace(const iqk_weights* w, int64_t T, int k, size_t* bytes);

/* Prefill with the dequantization fused into the MFMA grouped GEMM (the
 * two passes of "Surface" -- dequantize the stacked experts, then the
 * grouped GEMM -- in one kernel, without the dense copy): iqk_route, then
 * per expert the same bf16 weights iqk_dequant would write, rebuilt from
 * the compressed streams in registers and multiplied with the expert's
 * gathered bf16 token rows, float32 accumulation.  Arguments as
 * iqk_moe_prefill (workspace from iqk_moe_prefill_fused_workspace); the
 * value table may be any float32 values; the IQ1_S_R4 grid must be
 * ternary as for iqk_dequant's f16 / bf16 output (checked as the grid is
 * loaded: any other value makes every output row of the call NaN).  Widths: in = 512, 2048
 * or 4096 (IQK_E_WIDTH otherwise); out * iqk_row_bytes(fmt, in) < 2^31.
 * Accuracy: as iqk_moe_prefill (2e-2 against the float32-weight product;
 * the result differs from iqk_moe_prefill only in summation order). */
int iqk_moe_prefill_fused(const iqk_weights* w, const float* values, const int8_t* grid,
                          const void* x_bf16, int x_slots, const int32_t* ids, int64_t T, int k,
                          int sorted, void* workspace, size_t ws_bytes, float* y, void* stream);

/* Workspace of iqk_moe_prefill: the dense bf16 copy of all experts plus the
 * routing arrays, each rounded up to 256 bytes. */
int iqk_moe_prefill_workspace(const iqk_weights* w, int64_t T, int k, size_t* bytes);

/* Prefill ("Surface": many pairs): iqk_route, then iqk_dequant of all
 * experts to bf16 in the workspace ("dequantizes the stacked experts in one
 * kernel pass"), then iqk_grouped_gemm.  x: device bf16 [T, x_slots, in];
 * y: device float32 [T, k, out]; invalid ids give NaN rows.
 * Accuracy against the float32-weight product: ||y - y_exact|| /
 * ||y_exact|| <= 2e-2 (bf16 weights).  Invalid ids give NaN rows; the
 * output is float32 (an out_dtype argument is not provided). */
int iqk_moe_prefill(const iqk_weights* w, const float* values, const int8_t* grid,
                    const void* x_bf16, int x_slots, const int32_t* ids, int64_t T, int k,
                    int sorted, void* workspace, size_t ws_bytes, float* y, void* stream);

/* Measurement kernels for the deleted-decode address floor ("Pricing"
 * section: identical loads, decode removed, an integer accumulator reaching
 * the output).  iqk_floor_gemv issues the same loads as iqk_moe_gemv for the
 * same arguments (including the activation conversion), replaces the weight
 * decode with an integer XOR/add accumulator and writes one uint32 per
 * output element to `sink` (device [T, k, out]).  iqk_floor_dequant issues
 * the same loads and the same stores as iqk_dequant into `out` (device,
 * [nrows, in] of out_dtype) with the loaded words in place of the decoded
 * weights.  iqk_stream_read XOR-reduces `bytes` (a multiple of 16) of
 * device memory as a plain HBM streaming read and stores partial results
 * to sink[sink_words]. */
int iqk_floor_gemv(const iqk_weights* w, const float* values, const int8_t* grid,
                   const void* x, int x_dtype, int x_slots, const int32_t* ids,
                   int64_t T, int k, uint32_t* sink, void* stream);
int iqk_floor_dequant(const iqk_weights* w, int64_t row0, int64_t nrows, int out_dtype,
                      void* out, void* stream);
int iqk_stream_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words, void* stream);
/* Plain HBM streaming write (the write ceiling the dequantization producer
 * is measured against): `value` in every 32-bit word of `bytes` (a
 * multiple of 16) of device memory at `buf`, non-temporal 16-byte stores,
 * 1 KiB per wave and store instruction.  Each wave writes `runs` (1..16)
 * consecutive 1 KiB runs: 1 gives the highest plain write rate, 8 the store
 * shape of the bf16 producer (each wave stores the 8 KiB it decoded).
 * Other values of `runs` fail with IQK_E_ARG. */
int iqk_stream_write(void* buf, size_t bytes, uint32_t value, int runs, void* stream);

/* Message of the last failed call on this thread ("" if none). */
const char* iqk_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* IQK_H */
