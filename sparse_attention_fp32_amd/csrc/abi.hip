// Error plumbing and version of libdsa.
#include <stdlib.h>
#include <string.h>

#include "dsa_host.hpp"

namespace dsa {

static thread_local char g_err[512] = "";
static thread_local bool g_dry = false;

bool dry_run() { return g_dry; }
DryRun::DryRun() { g_dry = true; }
DryRun::~DryRun() { g_dry = false; }

dsa_status set_error(dsa_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_err[0] = '\0'; }

dsa_status check_launch(const char* what) {
  if (g_dry) return DSA_OK;  // nothing was launched
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return set_error(DSA_ERR_LAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return DSA_OK;
}

bool trace_enabled() {
  static int on = -1;
  if (on < 0) {
    const char* v = getenv("DSA_TRACE");
    on = (v && strcmp(v, "1") == 0) ? 1 : 0;
  }
  return on == 1;
}

}  // namespace dsa

DSA_EXPORT int dsa_abi_version(void) { return DSA_ABI_VERSION; }
DSA_EXPORT const char* dsa_last_error(void) { return dsa::g_err; }
