// Host-side helpers of libdsa: argument checks, thread-local error text,
// launch-status translation.  Every entry point validates before it launches.
#pragma once
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "dsa.h"

#define DSA_EXPORT extern "C" __attribute__((visibility("default")))

namespace dsa {

dsa_status set_error(dsa_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
// Reports a launch failure of `what` (hipGetLastError after the launch).
dsa_status check_launch(const char* what);
bool trace_enabled();

// Validation pass of a composite call (dsa_decode_step): while a DryRun is in
// scope on this thread, every entry point runs all of its argument checks and
// returns at the point where it would launch, with nothing enqueued.  Each
// launch site begins with `if (dsa::dry_run()) return DSA_OK;` after the last
// check of its call.
bool dry_run();
struct DryRun {
  DryRun();
  ~DryRun();
  DryRun(const DryRun&) = delete;
  DryRun& operator=(const DryRun&) = delete;
};

// True when every non-NULL pointer is 16-byte aligned (the kernels' vector
// loads and stores need it).
inline bool aligned16() { return true; }
template <typename P, typename... R>
inline bool aligned16(P p, R... rest) {
  return ((uintptr_t)(const void*)p & 15u) == 0 && aligned16(rest...);
}

}  // namespace dsa

#define DSA_REQUIRE(cond, code, ...)                  \
  do {                                                \
    if (!(cond)) return ::dsa::set_error(code, __VA_ARGS__); \
  } while (0)

// INVALID_ARG unless every listed (non-NULL) tensor pointer is 16-byte aligned.
#define DSA_REQUIRE_ALIGNED(who, ...)                                               \
  DSA_REQUIRE(::dsa::aligned16(__VA_ARGS__), DSA_ERR_INVALID_ARG,                   \
              "%s: a tensor pointer is not 16-byte aligned", who)
