// iqk_host.cpp -- C-ABI entry points of the IQ_K routed-expert library that
// run on the device: argument validation and dispatch to the HIP kernels
// (the host relayout is in iqk_relayout.cpp).  See include/iqk.h for the
// contract of every call and the byte layouts.
#include <algorithm>
#include <cmath>

#include "iqk_internal.h"
#include "iqk_status.h"

using iqk::check_fmt_shape;
using iqk::fail;
using iqk::known_fmt;
using iqk::ok;

namespace {

int hip_fail(hipError_t e, const char* where) {
    return fail(IQK_E_HIP, "%s: %s", where, hipGetErrorString(e));
}

int check_weights(const iqk_weights* w) {
    if (!w) return fail(IQK_E_ARG, "null weight descriptor");
    int rc = check_fmt_shape(w->fmt, w->in);
    if (rc) return rc;
    if (w->experts <= 0 || w->out <= 0) return fail(IQK_E_ARG, "experts and out must be positive");
    if (!w->streams) return fail(IQK_E_ARG, "null stream pointer");
    const int64_t R = w->experts * w->out;
    const size_t need = (size_t)(R * iqk::row_bytes(w->fmt, w->in));
    if (w->streams_bytes != need)
        return fail(IQK_E_SIZE, "streams_bytes %zu != %zu for %lld rows of %lld", w->streams_bytes, need,
                    (long long)R, (long long)w->in);
    return IQK_OK;
}

// Value table -> int8 m_i with values[i] = m_i * 2^e (common e).
bool table_to_int8(const float* v, uint32_t* lo, uint32_t* hi, float* scale) {
    int emin = 1 << 30;
    float amax = 0.f;
    for (int i = 0; i < 8; ++i) {
        if (!std::isfinite(v[i])) return false;
        if (v[i] == 0.f) continue;
        int ex;
        double m = std::frexp((double)v[i], &ex);  // v = m * 2^ex, 0.5 <= |m| < 1
        // lowest set bit of the 24-bit significand
        int64_t sig = (int64_t)std::ldexp(std::fabs(m), 24);
        int tz = 0;
        while ((sig & 1) == 0) { sig >>= 1; ++tz; }
        emin = std::min(emin, ex - 24 + tz);
        amax = std::max(amax, std::fabs(v[i]));
    }
    int e = (emin == (1 << 30)) ? 0 : emin;
    int8_t m[8];
    for (int i = 0; i < 8; ++i) {
        double q = std::ldexp((double)v[i], -e);
        if (std::fabs(q) > 127.0 || q != std::floor(q)) return false;
        m[i] = (int8_t)q;
    }
    (void)amax;
    *lo = (uint32_t)(uint8_t)m[0] | ((uint32_t)(uint8_t)m[1] << 8) | ((uint32_t)(uint8_t)m[2] << 16) | ((uint32_t)(uint8_t)m[3] << 24);
    *hi = (uint32_t)(uint8_t)m[4] | ((uint32_t)(uint8_t)m[5] << 8) | ((uint32_t)(uint8_t)m[6] << 16) | ((uint32_t)(uint8_t)m[7] << 24);
    *scale = (float)std::ldexp(1.0, e);
    return std::isfinite(*scale) && *scale != 0.f;
}

int check_gemv_args(const iqk_weights* w, const float* values, const int8_t* grid, const void* x, int x_dtype,
                    int x_slots, const int32_t* ids, int64_t T, int k, const void* y, iqk::GemvLaunch* L) {
    int rc = check_weights(w);
    if (rc) return rc;
    if (w->in != 512 && w->in != 2048 && w->in != 4096)
        return fail(IQK_E_WIDTH, "decode matvec has no instance for input width %lld (instances: 512, 2048, 4096)",
                    (long long)w->in);
    if (T < 0 || k <= 0) return fail(IQK_E_ARG, "T must be >= 0 and k > 0");
    if (T * k > 65535LL * 64) return fail(IQK_E_ARG, "T*k = %lld exceeds the decode limit", (long long)(T * k));
    if (x_slots != 1 && x_slots != k) return fail(IQK_E_ARG, "x_slots must be 1 or k");
    // the kernel indexes 4-row reduction groups of the whole call in 32 bits
    // one expert's plane, and one output row set, is addressed with 32-bit
    // byte offsets
    if (w->out * (int64_t)iqk::row_bytes(w->fmt, w->in) > 0x7FFFFFFFLL)
        return fail(IQK_E_ARG, "decode matvec needs out * row bytes < 2^31 (out = %lld)", (long long)w->out);
    if (T * k * ((w->out + 3) / 4) > 0x7FFFFFFFLL)
        return fail(IQK_E_ARG, "T*k*ceil(out/4) = %lld exceeds 2^31 - 1", (long long)(T * k * ((w->out + 3) / 4)));
    if (x_dtype != IQK_F32 && x_dtype != IQK_BF16) return fail(IQK_E_ARG, "x_dtype must be IQK_F32 or IQK_BF16");
    if (T > 0 && (!x || !ids || !y)) return fail(IQK_E_ARG, "null x, ids or output");
    L->fmt = w->fmt;
    L->E = w->experts;
    L->out = w->out;
    L->n = w->in;
    L->streams = (const uint8_t*)w->streams;
    L->pl = iqk::planes(w->fmt, w->experts * w->out, w->in);
    L->tab_lo = L->tab_hi = 0;
    L->tab_scale = 1.f;
    L->grid = grid;
    if (w->fmt == IQK_IQ1_S_R4) {
        if (!grid) return fail(IQK_E_ARG, "IQ1_S_R4 needs the device grid");
    } else {
        if (!values) return fail(IQK_E_ARG, "2-bit members need the host value table");
        if (!table_to_int8(values, &L->tab_lo, &L->tab_hi, &L->tab_scale))
            return fail(IQK_E_TABLE, "value table is not m_i * 2^e with |m_i| <= 127");
    }
    L->x = x;
    L->x_dtype = x_dtype;
    L->x_slots = x_slots;
    L->ids = ids;
    L->T = T;
    L->k = k;
    L->y = nullptr;
    L->sink = nullptr;
    L->mode = 0;
    L->h = nullptr;
    L->route_w = nullptr;
    return IQK_OK;
}

}  // namespace

extern "C" {

static int dequant_common(const iqk_weights* w, int64_t row0, int64_t nrows, const float* values, const int8_t* grid,
                          int out_dtype, void* out, void* stream, bool floor_variant) {
    int rc = check_weights(w);
    if (rc) return rc;
    const int64_t R = w->experts * w->out;
    if (row0 < 0 || nrows < 0 || row0 + nrows > R) return fail(IQK_E_ARG, "row range outside the tensor");
    if (out_dtype != IQK_F32 && out_dtype != IQK_F16 && out_dtype != IQK_BF16) return fail(IQK_E_ARG, "bad out_dtype");
    if (nrows > 0 && !out) return fail(IQK_E_ARG, "null output");
    iqk::DequantLaunch L;
    L.fmt = w->fmt;
    L.out_dtype = out_dtype;
    L.R = R;
    L.n = w->in;
    L.row0 = row0;
    L.nrows = nrows;
    L.streams = (const uint8_t*)w->streams;
    L.pl = iqk::planes(w->fmt, R, w->in);
    for (int i = 0; i < 8; ++i) L.values[i] = 0.f;
    L.grid = grid;
    L.out = out;
    if (!floor_variant) {
        if (w->fmt == IQK_IQ1_S_R4) {
            if (!grid) return fail(IQK_E_ARG, "IQ1_S_R4 needs the device grid");
        } else {
            if (!values) return fail(IQK_E_ARG, "2-bit members need the host value table");
            for (int i = 0; i < 8; ++i) L.values[i] = values[i];
        }
    }
    if (nrows == 0) return ok();
    hipError_t e = iqk::launch_dequant(L, floor_variant, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, floor_variant ? "floor dequant launch" : "dequant launch");
    return ok();
}

int iqk_dequant(const iqk_weights* w, int64_t row0, int64_t nrows, const float* values, const int8_t* grid,
                int out_dtype, void* out, void* stream) {
    return dequant_common(w, row0, nrows, values, grid, out_dtype, out, stream, false);
}

int iqk_floor_dequant(const iqk_weights* w, int64_t row0, int64_t nrows, int out_dtype, void* out, void* stream) {
    return dequant_common(w, row0, nrows, nullptr, nullptr, out_dtype, out, stream, true);
}

int iqk_moe_gemv(const iqk_weights* w, const float* values, const int8_t* grid, const void* x, int x_dtype,
                 int x_slots, const int32_t* ids, int64_t T, int k, float* y, void* stream) {
    iqk::GemvLaunch L;
    int rc = check_gemv_args(w, values, grid, x, x_dtype, x_slots, ids, T, k, y, &L);
    if (rc) return rc;
    L.y = y;
    if (T == 0) return ok();
    hipError_t e = iqk::launch_gemv(L, false, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "decode matvec launch");
    return ok();
}

int iqk_moe_gemv_swiglu(const iqk_weights* w, const float* values, const int8_t* grid, const void* x, int x_dtype,
                        int x_slots, const int32_t* ids, int64_t T, int k, uint16_t* h, void* stream) {
    iqk::GemvLaunch L;
    int rc = check_gemv_args(w, values, grid, x, x_dtype, x_slots, ids, T, k, h, &L);
    if (rc) return rc;
    if (w->out % 2) return fail(IQK_E_SHAPE, "SwiGLU needs an even number of gate/up rows (out = %lld)", (long long)w->out);
    L.mode = 1;
    L.h = h;
    if (T == 0) return ok();
    hipError_t e = iqk::launch_gemv(L, false, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "SwiGLU matvec launch");
    return ok();
}

int iqk_moe_gemv_combine(const iqk_weights* w, const float* values, const int8_t* grid, const void* x, int x_dtype,
                         int x_slots, const int32_t* ids, const float* route_w, int64_t T, int k, float* y,
                         void* stream) {
    iqk::GemvLaunch L;
    int rc = check_gemv_args(w, values, grid, x, x_dtype, x_slots, ids, T, k, y, &L);
    if (rc) return rc;
    if (k > 8) return fail(IQK_E_ARG, "combine handles at most 8 slots per token (k = %d)", k);
    if (T > 0 && !route_w) return fail(IQK_E_ARG, "null router weights");
    L.mode = 2;
    L.y = y;
    L.route_w = route_w;
    if (T == 0) return ok();
    hipError_t e = iqk::launch_gemv(L, false, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "combine matvec launch");
    return ok();
}

int iqk_floor_gemv(const iqk_weights* w, const float* values, const int8_t* grid, const void* x, int x_dtype,
                   int x_slots, const int32_t* ids, int64_t T, int k, uint32_t* sink, void* stream) {
    iqk::GemvLaunch L;
    int rc = check_gemv_args(w, values, grid, x, x_dtype, x_slots, ids, T, k, sink, &L);
    if (rc) return rc;
    L.sink = sink;
    if (T == 0) return ok();
    hipError_t e = iqk::launch_gemv(L, true, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "floor matvec launch");
    return ok();
}

int iqk_route(const int32_t* ids, int64_t P, int64_t E, int sorted, int32_t* counts, int32_t* offsets, int32_t* perm,
              void* stream) {
    if (P < 0 || P > (1LL << 24)) return fail(IQK_E_ARG, "pair count %lld outside [0, 2^24]", (long long)P);
    if (E <= 0 || E > 16384) return fail(IQK_E_ARG, "expert count %lld outside [1, 16384]", (long long)E);
    if (sorted != 0 && sorted != 1) return fail(IQK_E_ARG, "sorted must be 0 or 1");
    if (!counts || !offsets || (P > 0 && (!ids || !perm))) return fail(IQK_E_ARG, "null pointer");
    iqk::RouteLaunch L{ids, P, E, sorted, counts, offsets, perm};
    hipError_t e = iqk::launch_route(L, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "route launch");
    return ok();
}

int iqk_grouped_gemm(const void* W_bf16, int64_t E, int64_t out, int64_t in, const void* x_bf16, int x_slots,
                     int64_t T, int k, const int32_t* offsets, const int32_t* perm, float* y, void* stream) {
    if (E <= 0 || out <= 0 || in <= 0 || T < 0 || k <= 0) return fail(IQK_E_ARG, "bad sizes");
    if (in % 64) return fail(IQK_E_SHAPE, "grouped GEMM needs in %% 64 == 0");
    if (out % 16) return fail(IQK_E_SHAPE, "grouped GEMM needs out %% 16 == 0");
    if (x_slots != 1 && x_slots != k) return fail(IQK_E_ARG, "x_slots must be 1 or k");
    if (T * k > (1LL << 24)) return fail(IQK_E_ARG, "too many pairs");
    if (!W_bf16 || !offsets || (T > 0 && (!x_bf16 || !perm || !y))) return fail(IQK_E_ARG, "null pointer");
    if (T == 0) return ok();
    iqk::GemmLaunch L{W_bf16, E, out, in, x_bf16, x_slots, T, k, offsets, perm, y};
    hipError_t e = iqk::launch_grouped_gemm(L, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "grouped GEMM launch");
    return ok();
}

static size_t round256(size_t b) { return (b + 255) / 256 * 256; }

int iqk_moe_prefill_workspace(const iqk_weights* w, int64_t T, int k, size_t* bytes) {
    if (!w || !bytes) return fail(IQK_E_ARG, "null pointer");
    int rc = check_fmt_shape(w->fmt, w->in);
    if (rc) return rc;
    if (w->experts <= 0 || w->out <= 0 || T < 0 || k <= 0) return fail(IQK_E_ARG, "bad sizes");
    const int64_t P = T * k;
    *bytes = round256((size_t)(w->experts * w->out * w->in) * 2) + round256((size_t)w->experts * 4) +
             round256((size_t)(w->experts + 1) * 4) + round256((size_t)std::max<int64_t>(P, 1) * 4);
    return ok();
}

int iqk_moe_prefill(const iqk_weights* w, const float* values, const int8_t* grid, const void* x_bf16, int x_slots,
                    const int32_t* ids, int64_t T, int k, int sorted, void* workspace, size_t ws_bytes, float* y,
                    void* stream) {
    int rc = check_weights(w);
    if (rc) return rc;
    if (T < 0 || k <= 0) return fail(IQK_E_ARG, "T must be >= 0 and k > 0");
    if (T * k > (1LL << 24)) return fail(IQK_E_ARG, "too many pairs");
    if (x_slots != 1 && x_slots != k) return fail(IQK_E_ARG, "x_slots must be 1 or k");
    if (sorted != 0 && sorted != 1) return fail(IQK_E_ARG, "sorted must be 0 or 1");
    if (w->out % 16) return fail(IQK_E_SHAPE, "prefill needs out %% 16 == 0");
    if (w->in % 64) return fail(IQK_E_SHAPE, "prefill needs in %% 64 == 0");
    if (w->experts > 16384) return fail(IQK_E_ARG, "prefill routing supports at most 16384 experts");
    if (w->fmt == IQK_IQ1_S_R4 ? !grid : !values) return fail(IQK_E_ARG, "missing value table or grid");
    size_t need = 0;
    rc = iqk_moe_prefill_workspace(w, T, k, &need);
    if (rc) return rc;
    if (!workspace || ws_bytes < need) return fail(IQK_E_SIZE, "workspace needs %zu bytes (got %zu)", need, ws_bytes);
    if (T > 0 && (!x_bf16 || !ids || !y)) return fail(IQK_E_ARG, "null x, ids or output");
    if (T == 0) return ok();
    const int64_t E = w->experts, P = T * k;
    uint8_t* ws = (uint8_t*)workspace;
    void* dense = ws;
    ws += round256((size_t)(E * w->out * w->in) * 2);
    int32_t* counts = (int32_t*)ws;
    ws += round256((size_t)E * 4);
    int32_t* offsets = (int32_t*)ws;
    ws += round256((size_t)(E + 1) * 4);
    int32_t* perm = (int32_t*)ws;
    hipStream_t s = (hipStream_t)stream;
    iqk::RouteLaunch RL{ids, P, E, sorted, counts, offsets, perm};
    RL.ynan = y;  // rows of pairs with an invalid id: NaN, as on the per-pair path
    RL.yout = w->out;
    hipError_t e = iqk::launch_route(RL, s);
    if (e != hipSuccess) return hip_fail(e, "prefill route launch");
    rc = iqk_dequant(w, 0, E * w->out, values, grid, IQK_BF16, dense, stream);
    if (rc) return rc;
    iqk::GemmLaunch GL{dense, E, w->out, w->in, x_bf16, x_slots, T, k, offsets, perm, y};
    e = iqk::launch_grouped_gemm(GL, s);
    if (e != hipSuccess) return hip_fail(e, "prefill grouped GEMM launch");
    return ok();
}

int iqk_moe_prefill_fused_workspace(const iqk_weights* w, int64_t T, int k, size_t* bytes) {
    if (!w || !bytes) return fail(IQK_E_ARG, "null pointer");
    int rc = check_fmt_shape(w->fmt, w->in);
    if (rc) return rc;
    if (w->experts <= 0 || w->out <= 0 || T < 0 || k <= 0) return fail(IQK_E_ARG, "bad sizes");
    const int64_t P = T * k;
    *bytes = round256((size_t)w->experts * 4) + round256((size_t)(w->experts + 1) * 4) +
             round256((size_t)std::max<int64_t>(P, 1) * 4) + round256((size_t)(w->experts + 1) * 8);
    return ok();
}

int iqk_moe_prefill_fused(const iqk_weights* w, const float* values, const int8_t* grid, const void* x_bf16,
                          int x_slots, const int32_t* ids, int64_t T, int k, int sorted, void* workspace,
                          size_t ws_bytes, float* y, void* stream) {
    int rc = check_weights(w);
    if (rc) return rc;
    if (w->in != 512 && w->in != 2048 && w->in != 4096)
        return fail(IQK_E_WIDTH, "fused prefill has no instance for input width %lld (instances: 512, 2048, 4096)",
                    (long long)w->in);
    if (T < 0 || k <= 0) return fail(IQK_E_ARG, "T must be >= 0 and k > 0");
    if (T * k > (1LL << 24)) return fail(IQK_E_ARG, "too many pairs");
    if (x_slots != 1 && x_slots != k) return fail(IQK_E_ARG, "x_slots must be 1 or k");
    if (sorted != 0 && sorted != 1) return fail(IQK_E_ARG, "sorted must be 0 or 1");
    if (w->experts > 16384) return fail(IQK_E_ARG, "prefill routing supports at most 16384 experts");
    if (w->out * (int64_t)iqk::row_bytes(w->fmt, w->in) > 0x7FFFFFFFLL)
        return fail(IQK_E_ARG, "fused prefill needs out * row bytes < 2^31 (out = %lld)", (long long)w->out);
    if (T * k * w->out * 4 > 0x7FFFFFFFLL)
        return fail(IQK_E_ARG, "fused prefill needs T * k * out * 4 < 2^31");
    if (w->fmt == IQK_IQ1_S_R4 ? !grid : !values) return fail(IQK_E_ARG, "missing value table or grid");
    size_t need = 0;
    rc = iqk_moe_prefill_fused_workspace(w, T, k, &need);
    if (rc) return rc;
    if (!workspace || ws_bytes < need) return fail(IQK_E_SIZE, "workspace needs %zu bytes (got %zu)", need, ws_bytes);
    if (T > 0 && (!x_bf16 || !ids || !y)) return fail(IQK_E_ARG, "null x, ids or output");
    if (T == 0) return ok();
    const int64_t E = w->experts, P = T * k;
    uint8_t* ws = (uint8_t*)workspace;
    int32_t* counts = (int32_t*)ws;
    ws += round256((size_t)E * 4);
    int32_t* offsets = (int32_t*)ws;
    ws += round256((size_t)(E + 1) * 4);
    int32_t* perm = (int32_t*)ws;
    ws += round256((size_t)P * 4);
    int64_t* plan = (int64_t*)ws;
    hipStream_t s = (hipStream_t)stream;
    iqk::RouteLaunch RL{ids, P, E, sorted, counts, offsets, perm};
    RL.ynan = y;  // rows of pairs with an invalid id: NaN, as on the per-pair path
    RL.yout = w->out;
    hipError_t e = iqk::launch_route(RL, s);
    if (e != hipSuccess) return hip_fail(e, "prefill route launch");
    iqk::FusedLaunch FL;
    FL.fmt = w->fmt;
    FL.E = E;
    FL.out = w->out;
    FL.n = w->in;
    FL.streams = (const uint8_t*)w->streams;
    FL.pl = iqk::planes(w->fmt, E * w->out, w->in);
    FL.values = values;
    FL.grid = grid;
    FL.x = x_bf16;
    FL.x_slots = x_slots;
    FL.k = k;
    FL.T = T;
    FL.offsets = offsets;
    FL.perm = perm;
    FL.plan = plan;
    FL.y = y;
    e = iqk::launch_fused_prefill(FL, s);
    if (e != hipSuccess) return hip_fail(e, "fused prefill launch");
    return ok();
}

int iqk_moe_gemv_grouped_workspace(const iqk_weights* w, int64_t T, int k, size_t* bytes) {
    if (!w || !bytes) return fail(IQK_E_ARG, "null pointer");
    int rc = check_fmt_shape(w->fmt, w->in);
    if (rc) return rc;
    if (w->experts <= 0 || w->out <= 0 || T < 0 || k <= 0) return fail(IQK_E_ARG, "bad sizes");
    const int64_t P = T * k;
    *bytes = round256((size_t)w->experts * 4) + round256((size_t)(w->experts + 1) * 4) +
             round256((size_t)std::max<int64_t>(P, 1) * 4) + round256((size_t)(w->experts + 1) * 8);
    return ok();
}

int iqk_moe_gemv_grouped(const iqk_weights* w, const float* values, const int8_t* grid, const void* x, int x_dtype,
                         int x_slots, const int32_t* ids, int64_t T, int k, int sorted, void* workspace,
                         size_t ws_bytes, float* y, void* stream) {
    iqk::GemvLaunch L;
    int rc = check_gemv_args(w, values, grid, x, x_dtype, x_slots, ids, T, k, y, &L);
    if (rc) return rc;
    if (sorted != 0 && sorted != 1) return fail(IQK_E_ARG, "sorted must be 0 or 1");
    if (w->experts > 16384) return fail(IQK_E_ARG, "routing supports at most 16384 experts");
    if (T * k * w->out * 4 > 0x7FFFFFFFLL) return fail(IQK_E_ARG, "grouped matvec needs T * k * out * 4 < 2^31");
    size_t need = 0;
    rc = iqk_moe_gemv_grouped_workspace(w, T, k, &need);
    if (rc) return rc;
    if (!workspace || ws_bytes < need) return fail(IQK_E_SIZE, "workspace needs %zu bytes (got %zu)", need, ws_bytes);
    if (T == 0) return ok();
    L.y = y;
    const int64_t E = w->experts, P = T * k;
    uint8_t* ws = (uint8_t*)workspace;
    int32_t* counts = (int32_t*)ws;
    ws += round256((size_t)E * 4);
    int32_t* offsets = (int32_t*)ws;
    ws += round256((size_t)(E + 1) * 4);
    int32_t* perm = (int32_t*)ws;
    ws += round256((size_t)P * 4);
    int64_t* plan = (int64_t*)ws;
    hipStream_t s = (hipStream_t)stream;
    iqk::RouteLaunch RL{ids, P, E, sorted, counts, offsets, perm};
    RL.ynan = y;  // rows of pairs with an invalid id: NaN, as on the per-pair path
    RL.yout = w->out;
    hipError_t e = iqk::launch_route(RL, s);
    if (e != hipSuccess) return hip_fail(e, "grouped matvec route launch");
    e = iqk::launch_gemv_grouped(L, offsets, perm, plan, s);
    if (e != hipSuccess) return hip_fail(e, "grouped matvec launch");
    return ok();
}

int iqk_moe_auto_workspace(const iqk_weights* w, int64_t T, int k, size_t* bytes) {
    // the grouped matvec and the fused prefill need the same routing arrays and plan
    return iqk_moe_gemv_grouped_workspace(w, T, k, bytes);
}

int iqk_moe_auto(const iqk_weights* w, const float* values, const int8_t* grid, const void* x, int x_dtype,
                 int x_slots, const int32_t* ids, int64_t T, int k, void* workspace, size_t ws_bytes, float* y,
                 int* path, void* stream) {
    int rc = check_weights(w);
    if (rc) return rc;
    if (T < 0 || k <= 0) return fail(IQK_E_ARG, "T must be >= 0 and k > 0");
    // measured crossover on the routed geometry (top-6 of 256 experts): with
    // in = 4096 the per-pair matvec up to 32 tokens (3/4 pair per expert),
    // the grouped matvec up to 64 (3/2), the fused prefill beyond; with a
    // narrower input the per-pair matvec up to 32 tokens (3/4), then the
    // fused prefill
    const double per_expert = (double)(T * k) / (double)w->experts;
    const double lim_pair = 0.75;
    const double lim_grouped = w->in >= 4096 ? 1.5 : 0.75;
    uint32_t lo = 0, hi = 0;
    float sc = 1.f;
    const bool int8_table = w->fmt == IQK_IQ1_S_R4 || (values && table_to_int8(values, &lo, &hi, &sc));
    int choice = per_expert <= lim_pair ? 0 : (per_expert <= lim_grouped ? 1 : 2);
    if (choice == 2 && x_dtype != IQK_BF16) choice = 1;  // the prefill takes bf16 activations
    if (choice < 2 && !int8_table && x_dtype == IQK_BF16) choice = 2;  // any float table: the prefill
    if (path) *path = choice;
    if (choice == 0) return iqk_moe_gemv(w, values, grid, x, x_dtype, x_slots, ids, T, k, y, stream);
    if (choice == 1)
        return iqk_moe_gemv_grouped(w, values, grid, x, x_dtype, x_slots, ids, T, k, 0, workspace, ws_bytes, y,
                                    stream);
    return iqk_moe_prefill_fused(w, values, grid, x, x_slots, ids, T, k, 0, workspace, ws_bytes, y, stream);
}

int iqk_swiglu(const float* y_gu, int64_t P, int64_t I, uint16_t* h, void* stream) {
    if (P < 0 || I <= 0) return fail(IQK_E_ARG, "bad sizes");
    if (I % 4) return fail(IQK_E_SHAPE, "SwiGLU needs I %% 4 == 0 (I = %lld)", (long long)I);
    if (P == 0) return ok();
    if (!y_gu || !h) return fail(IQK_E_ARG, "null pointer");
    if ((uintptr_t)y_gu % 16 || (uintptr_t)h % 8) return fail(IQK_E_ARG, "y_gu must be 16-byte and h 8-byte aligned");
    hipError_t e = iqk::launch_swiglu(y_gu, P, I, h, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "SwiGLU launch");
    return ok();
}

int iqk_combine(const float* y, const float* route_w, int64_t T, int k, int64_t out, float* yc, void* stream) {
    if (T < 0 || k <= 0 || out <= 0) return fail(IQK_E_ARG, "bad sizes");
    if (out % 4) return fail(IQK_E_SHAPE, "combine needs out %% 4 == 0 (out = %lld)", (long long)out);
    if (T == 0) return ok();
    if (!y || !route_w || !yc) return fail(IQK_E_ARG, "null pointer");
    if ((uintptr_t)y % 16 || (uintptr_t)yc % 16) return fail(IQK_E_ARG, "y and yc must be 16-byte aligned");
    hipError_t e = iqk::launch_combine(y, route_w, T, k, out, yc, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    return ok();
}

int iqk_stream_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words, void* stream) {
    if (!buf || !sink || bytes == 0 || bytes % 16 || sink_words == 0) return fail(IQK_E_ARG, "bad stream-read arguments");
    hipError_t e = iqk::launch_stream_read(buf, bytes, sink, sink_words, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "stream read launch");
    return ok();
}

int iqk_stream_write(void* buf, size_t bytes, uint32_t value, int runs, void* stream) {
    if (!buf || bytes == 0 || bytes % 16 || runs < 1 || runs > 16) return fail(IQK_E_ARG, "bad stream-write arguments");
    hipError_t e = iqk::launch_stream_write(buf, bytes, value, runs, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "stream write launch");
    return ok();
}


}  // extern "C"
