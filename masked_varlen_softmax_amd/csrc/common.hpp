// common.hpp - status codes, error reporting and small helpers shared by the
// host-side C++ and the HIP sources of libmvs.
#pragma once

#include <cstdint>

#include "mvs.h"

#if defined(__HIPCC__)
#define MVS_HD __host__ __device__
#else
#define MVS_HD
#endif

namespace mvs {

// Stores a printf-style message for mvs_last_error() on this thread and
// returns `code`, so validation can `return fail(MVS_ERR_INVALID, "...")`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

inline bool aligned_to(const void* p, uintptr_t bytes) { return (reinterpret_cast<uintptr_t>(p) % bytes) == 0; }

}  // namespace mvs
