// iqk_relayout.cpp -- the host relayout between the ik wire blocks and the
// canonical per-row streams, and the layout queries of the C ABI.
// Plain C++ (no HIP), so the CPU tests also build it with sanitizers.
//
// "mlx-iqk" package description, introduction (the relayout at build time
// that makes the values consumed along k contiguous, changing no value and
// no stored byte budget) and "Format" (stream tables, row budgets, the
// IQ1_S_R4 wire in four-row groups).  The wire bit positions are the
// stand-in reading documented in iqk.h.
#include <algorithm>
#include <cstring>
#include <thread>
#include <vector>

#include "iqk_layout.h"
#include "iqk_status.h"

using iqk::check_fmt_shape;
using iqk::fail;
using iqk::known_fmt;
using iqk::ok;

namespace {

// ---------------------------------------------------------------------------
// Host relayout.  Wire layouts are the stand-in readings of the ik block
// structs documented in iqk.h; the stream layout is the canonical one.
// ---------------------------------------------------------------------------

inline uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }
inline void wr16(uint8_t* p, uint16_t v) {
    p[0] = (uint8_t)v;
    p[1] = (uint8_t)(v >> 8);
}

// Codes of one 256-weight block: wire qs[64] (interleaved) <-> k-contiguous
// qs[64] (weight j at byte j/4, bits 2(j%4)).  Wire weight j = 128h + 32p + l
// sits in byte 32h + l at bits 2p.
inline void qs_wire_to_stream(const uint8_t* wq, uint8_t* sq) {
    for (int m = 0; m < 64; ++m) {
        const int j0 = 4 * m, h = j0 / 128, p = (j0 % 128) / 32, l0 = j0 % 32;
        const uint8_t* src = wq + 32 * h + l0;
        const int sh = 2 * p;
        sq[m] = (uint8_t)(((src[0] >> sh) & 3) | (((src[1] >> sh) & 3) << 2) | (((src[2] >> sh) & 3) << 4) |
                          (((src[3] >> sh) & 3) << 6));
    }
}
inline void qs_stream_to_wire(const uint8_t* sq, uint8_t* wq) {
    std::memset(wq, 0, 64);
    for (int m = 0; m < 64; ++m) {
        const int j0 = 4 * m, h = j0 / 128, p = (j0 % 128) / 32, l0 = j0 % 32;
        uint8_t* dst = wq + 32 * h + l0;
        const int sh = 2 * p;
        for (int i = 0; i < 4; ++i) dst[i] |= (uint8_t)(((sq[m] >> (2 * i)) & 3) << sh);
    }
}

struct Relayout {
    int fmt;
    int64_t R, n;
    iqk::Planes pl;
};

// One row (IQ2_*) or one four-row group (IQ1_S_R4), wire -> streams.
void pack_unit(const Relayout& L, const uint8_t* wire, uint8_t* s, int64_t u) {
    const int64_t n = L.n, R = L.R;
    if (L.fmt == IQK_IQ2_KS) {
        const int64_t r = u;
        const uint8_t* row = wire + r * iqk::row_bytes(L.fmt, n);
        uint8_t* qs = s + L.pl.off[0] + r * n / 4;
        uint8_t* scl = s + L.pl.off[1] + r * n / 64;
        uint8_t* sch = s + L.pl.off[2] + r * n / 256;
        uint8_t* sex = s + L.pl.off[3] + r * n / 256;
        wr16(s + L.pl.off[4] + 2 * r, rd16(row));
        for (int64_t b = 0; b < n / 256; ++b) {
            const uint8_t* blk = row + 2 + 70 * b;
            const uint16_t extra = rd16(blk);
            sex[b] = (uint8_t)(extra & 0xff);
            sch[b] = (uint8_t)(extra >> 8);
            std::memcpy(scl + 4 * b, blk + 2, 4);
            qs_wire_to_stream(blk + 6, qs + 64 * b);
        }
    } else if (L.fmt == IQK_IQ2_K) {
        const int64_t r = u;
        const uint8_t* row = wire + r * iqk::row_bytes(L.fmt, n);
        uint8_t* qs = s + L.pl.off[0] + r * n / 4;
        uint8_t* scl = s + L.pl.off[1] + r * n / 32;
        uint8_t* sex = s + L.pl.off[2] + r * n / 128;
        uint8_t* dv = s + L.pl.off[3] + r * (n / 256) * 2;
        for (int64_t b = 0; b < n / 256; ++b) {
            const uint8_t* blk = row + 76 * b;
            wr16(dv + 2 * b, rd16(blk));
            wr16(sex + 2 * b, rd16(blk + 2));
            std::memcpy(scl + 8 * b, blk + 4, 8);
            qs_wire_to_stream(blk + 12, qs + 64 * b);
        }
    } else {
        const int64_t g = u, rb = iqk::row_bytes(L.fmt, n);
        const uint8_t* grp = wire + g * 4 * rb;
        for (int ri = 0; ri < 4; ++ri) {
            const int64_t r = 4 * g + ri;
            uint8_t* qs = s + L.pl.off[0] + r * n / 8;
            uint8_t* qh = s + L.pl.off[1] + r * (n / 32) * 2;
            wr16(s + L.pl.off[2] + 2 * r, rd16(grp + 2 * ri));
            for (int64_t b = 0; b < n / 32; ++b) {
                const uint8_t* blk = grp + 8 + 24 * b;
                for (int j = 0; j < 4; ++j) qs[4 * b + j] = blk[4 * j + ri];
                wr16(qh + 2 * b, rd16(blk + 16 + 2 * ri));
            }
        }
    }
    (void)R;
}

void unpack_unit(const Relayout& L, const uint8_t* s, uint8_t* wire, int64_t u) {
    const int64_t n = L.n;
    if (L.fmt == IQK_IQ2_KS) {
        const int64_t r = u;
        uint8_t* row = wire + r * iqk::row_bytes(L.fmt, n);
        const uint8_t* qs = s + L.pl.off[0] + r * n / 4;
        const uint8_t* scl = s + L.pl.off[1] + r * n / 64;
        const uint8_t* sch = s + L.pl.off[2] + r * n / 256;
        const uint8_t* sex = s + L.pl.off[3] + r * n / 256;
        wr16(row, rd16(s + L.pl.off[4] + 2 * r));
        for (int64_t b = 0; b < n / 256; ++b) {
            uint8_t* blk = row + 2 + 70 * b;
            wr16(blk, (uint16_t)(sex[b] | (sch[b] << 8)));
            std::memcpy(blk + 2, scl + 4 * b, 4);
            qs_stream_to_wire(qs + 64 * b, blk + 6);
        }
    } else if (L.fmt == IQK_IQ2_K) {
        const int64_t r = u;
        uint8_t* row = wire + r * iqk::row_bytes(L.fmt, n);
        const uint8_t* qs = s + L.pl.off[0] + r * n / 4;
        const uint8_t* scl = s + L.pl.off[1] + r * n / 32;
        const uint8_t* sex = s + L.pl.off[2] + r * n / 128;
        const uint8_t* dv = s + L.pl.off[3] + r * (n / 256) * 2;
        for (int64_t b = 0; b < n / 256; ++b) {
            uint8_t* blk = row + 76 * b;
            wr16(blk, rd16(dv + 2 * b));
            wr16(blk + 2, rd16(sex + 2 * b));
            std::memcpy(blk + 4, scl + 8 * b, 8);
            qs_stream_to_wire(qs + 64 * b, blk + 12);
        }
    } else {
        const int64_t g = u, rb = iqk::row_bytes(L.fmt, n);
        uint8_t* grp = wire + g * 4 * rb;
        for (int ri = 0; ri < 4; ++ri) {
            const int64_t r = 4 * g + ri;
            const uint8_t* qs = s + L.pl.off[0] + r * n / 8;
            const uint8_t* qh = s + L.pl.off[1] + r * (n / 32) * 2;
            wr16(grp + 2 * ri, rd16(s + L.pl.off[2] + 2 * r));
            for (int64_t b = 0; b < n / 32; ++b) {
                uint8_t* blk = grp + 8 + 24 * b;
                for (int j = 0; j < 4; ++j) blk[4 * j + ri] = qs[4 * b + j];
                wr16(blk + 16 + 2 * ri, rd16(qh + 2 * b));
            }
        }
    }
}

template <class F>
void parallel_units(int64_t units, F&& f) {
    unsigned hw = std::thread::hardware_concurrency();
    int64_t nt = std::min<int64_t>(std::max(1u, std::min(hw, 16u)), std::max<int64_t>(1, units / 64));
    if (nt <= 1) {
        for (int64_t u = 0; u < units; ++u) f(u);
        return;
    }
    std::vector<std::thread> th;
    for (int64_t t = 0; t < nt; ++t) {
        th.emplace_back([&, t] {
            const int64_t a = units * t / nt, b = units * (t + 1) / nt;
            for (int64_t u = a; u < b; ++u) f(u);
        });
    }
    for (auto& x : th) x.join();
}

int check_relayout(int fmt, const void* a, size_t a_bytes, int64_t rows, int64_t n, const void* b, size_t b_bytes) {
    int rc = check_fmt_shape(fmt, n);
    if (rc) return rc;
    if (rows < 0) return fail(IQK_E_ARG, "negative row count");
    if (fmt == IQK_IQ1_S_R4 && rows % 4) return fail(IQK_E_ROWS4, "IQ1_S_R4 wire needs rows %% 4 == 0 (got %lld)", (long long)rows);
    const size_t need = (size_t)(rows * iqk::row_bytes(fmt, n));
    if (a_bytes != need || b_bytes != need)
        return fail(IQK_E_SIZE, "relayout buffers must hold %zu bytes (got %zu and %zu)", need, a_bytes, b_bytes);
    if (need && (!a || !b)) return fail(IQK_E_ARG, "null buffer");
    const uint8_t* pa = (const uint8_t*)a;
    const uint8_t* pb = (const uint8_t*)b;
    if (need && pa < pb + need && pb < pa + need) return fail(IQK_E_ARG, "relayout buffers overlap");
    return IQK_OK;
}

}  // namespace

extern "C" {

size_t iqk_row_bytes(int fmt, int64_t n) {
    if (!known_fmt(fmt) || !iqk::shape_ok(fmt, n)) return 0;
    return (size_t)iqk::row_bytes(fmt, n);
}

int iqk_plane_offsets(int fmt, int64_t rows, int64_t n, int64_t off[5], int64_t* total) {
    int rc = check_fmt_shape(fmt, n);
    if (rc) return rc;
    if (rows < 0 || !off || !total) return fail(IQK_E_ARG, "bad rows or null output");
    iqk::Planes p = iqk::planes(fmt, rows, n);
    for (int i = 0; i < 5; ++i) off[i] = p.off[i];
    *total = p.total;
    return ok();
}

int iqk_pack_relayout(int fmt, const uint8_t* wire, size_t wire_bytes, int64_t rows, int64_t n, uint8_t* streams,
                      size_t streams_bytes) {
    int rc = check_relayout(fmt, wire, wire_bytes, rows, n, streams, streams_bytes);
    if (rc) return rc;
    Relayout L{fmt, rows, n, iqk::planes(fmt, rows, n)};
    const int64_t units = fmt == IQK_IQ1_S_R4 ? rows / 4 : rows;
    parallel_units(units, [&](int64_t u) { pack_unit(L, wire, streams, u); });
    return ok();
}

int iqk_unpack_relayout(int fmt, const uint8_t* streams, size_t streams_bytes, int64_t rows, int64_t n, uint8_t* wire,
                        size_t wire_bytes) {
    int rc = check_relayout(fmt, streams, streams_bytes, rows, n, wire, wire_bytes);
    if (rc) return rc;
    Relayout L{fmt, rows, n, iqk::planes(fmt, rows, n)};
    const int64_t units = fmt == IQK_IQ1_S_R4 ? rows / 4 : rows;
    parallel_units(units, [&](int64_t u) { unpack_unit(L, streams, wire, u); });
    return ok();
}

}  // extern "C"
