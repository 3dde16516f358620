// Host-side helpers of libdsa: argument checks, thread-local error text,
// launch-status translation.  Every entry point validates before it launches.
#pragma once
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include "dsa.h"

#define DSA_EXPORT extern "C" __attribute__((visibility("default")))

namespace dsa {

dsa_status set_error(dsa_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
// Reports a launch failure of `what` (hipGetLastError after the launch).
dsa_status check_launch(const char* what);
bool trace_enabled();

}  // namespace dsa

#define DSA_REQUIRE(cond, code, ...)                  \
  do {                                                \
    if (!(cond)) return ::dsa::set_error(code, __VA_ARGS__); \
  } while (0)
