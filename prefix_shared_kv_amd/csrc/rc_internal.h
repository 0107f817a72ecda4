// Internal helpers shared by the host and HIP translation units.
#pragma once

#include <cstdarg>
#include <cstdint>

#include "rc.h"

namespace rc {

// Set the thread-local error text and return `st`.
rc_status fail(rc_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Validate an rc_shape; returns RC_OK or the failure (with the error text set).
rc_status check_shape(const rc_shape* s);

inline int dtype_bytes(int32_t dt) { return dt == RC_F32 ? 4 : 2; }

}  // namespace rc
