// Host-side helpers of the C ABI: error reporting, argument checks, launch
// checks and device queries.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bloom_kernels.h"

namespace bloom {

// Records a thread-local message for bloom_last_error() and returns `s`.
bloom_status fail(bloom_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks hipGetLastError() after a launch.
bloom_status launch_status(const char* what);

// Compute units of the current device (cached per device).
int device_cu_count();

}  // namespace bloom

// Argument-check helpers: each returns from the calling entry point.
#define BLOOM_REQUIRE_PTR(p)                                                    \
  do {                                                                          \
    if ((p) == nullptr) return ::bloom::fail(BLOOM_ERR_NULL, "%s is NULL", #p); \
    if (!::bloom::aligned16(p))                                                 \
      return ::bloom::fail(BLOOM_ERR_ALIGN, "%s is not 16-byte aligned", #p);   \
  } while (0)

#define BLOOM_REQUIRE(cond, status, ...)                      \
  do {                                                        \
    if (!(cond)) return ::bloom::fail(status, __VA_ARGS__);   \
  } while (0)
