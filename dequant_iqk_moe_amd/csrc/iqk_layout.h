// iqk_layout.h -- byte layout of the canonical stream tensors (the
// "served relayout"), shared by the host relayout and the kernel launchers.
// Plain C++: no HIP, so the host relayout also builds without the HIP
// toolchain (the sanitizer builds of the CPU tests).
//
// "mlx-iqk" package description, "Format": the per-row streams of each
// member (IQ2_KS qs/scl/sch/sex/dv, IQ2_K qs/scl/sex/dv, IQ1_S_R4 qs/qh/dv)
// and the row budgets 2 + 70n/256, 76n/256 and 2 + 6n/32 bytes; here each
// stream is one plane over all rows of the stacked tensor.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/iqk.h"

namespace iqk {

// Plane byte offsets of an R-row canonical stream tensor (see iqk.h).
struct Planes {
    int64_t off[5];
    int64_t total;
};

inline bool shape_ok(int fmt, int64_t n) {
    if (n <= 0) return false;
    if (fmt == IQK_IQ2_KS || fmt == IQK_IQ2_K) return n % 256 == 0;
    if (fmt == IQK_IQ1_S_R4) return n % 32 == 0;
    return false;
}

inline int64_t row_bytes(int fmt, int64_t n) {
    if (fmt == IQK_IQ2_KS) return 2 + 70 * n / 256;
    if (fmt == IQK_IQ2_K) return 76 * n / 256;
    return 2 + 6 * n / 32;
}

inline Planes planes(int fmt, int64_t R, int64_t n) {
    Planes p;
    for (int i = 0; i < 5; ++i) p.off[i] = -1;
    if (fmt == IQK_IQ2_KS) {
        p.off[0] = 0;                       // qs
        p.off[1] = p.off[0] + R * n / 4;    // scl
        p.off[2] = p.off[1] + R * n / 64;   // sch
        p.off[3] = p.off[2] + R * n / 256;  // sex
        p.off[4] = p.off[3] + R * n / 256;  // dv
    } else if (fmt == IQK_IQ2_K) {
        p.off[0] = 0;                       // qs
        p.off[1] = p.off[0] + R * n / 4;    // scl
        p.off[2] = p.off[1] + R * n / 32;   // sex
        p.off[3] = p.off[2] + R * n / 128;  // dv
    } else {
        p.off[0] = 0;                       // qs
        p.off[1] = p.off[0] + R * n / 8;    // qh
        p.off[2] = p.off[1] + R * (n / 32) * 2;  // dv
    }
    p.total = R * row_bytes(fmt, n);
    return p;
}

}  // namespace iqk
