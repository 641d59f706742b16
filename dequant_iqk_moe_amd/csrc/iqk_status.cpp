// iqk_status.cpp -- per-thread error message and shared argument checks.
#include "iqk_status.h"

#include <cstdarg>
#include <cstdio>
#include <string>

#include "iqk_layout.h"

namespace {
thread_local std::string g_err;
}  // namespace

namespace iqk {


int fail(int code, const char* fmt_msg, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt_msg);
    vsnprintf(buf, sizeof buf, fmt_msg, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int ok() {
    g_err.clear();
    return IQK_OK;
}

bool known_fmt(int fmt) { return fmt == IQK_IQ2_KS || fmt == IQK_IQ2_K || fmt == IQK_IQ1_S_R4; }

int check_fmt_shape(int fmt, int64_t n) {
    if (!known_fmt(fmt)) return fail(IQK_E_FORMAT, "unknown format %d", fmt);
    if (!iqk::shape_ok(fmt, n))
        return fail(IQK_E_SHAPE, "in_features %lld violates the %s rule", (long long)n,
                    fmt == IQK_IQ1_S_R4 ? "multiple-of-32" : "multiple-of-256");
    return IQK_OK;
}

}  // namespace iqk

extern "C" const char* iqk_last_error(void) { return g_err.c_str(); }
