// iqk_status.h -- the per-thread error message behind iqk_last_error() and
// the argument checks shared by the host entry points.  Plain C++ (no HIP).
#pragma once

#include <stdint.h>

#include "../../include/iqk.h"

namespace iqk {

// Sets the calling thread's error message and returns `code`.
int fail(int code, const char* fmt_msg, ...) __attribute__((format(printf, 2, 3)));
// Clears the message and returns IQK_OK.
int ok();
bool known_fmt(int fmt);
// IQK_E_FORMAT for an unknown format, IQK_E_SHAPE when n breaks its width rule.
int check_fmt_shape(int fmt, int64_t n);

}  // namespace iqk
