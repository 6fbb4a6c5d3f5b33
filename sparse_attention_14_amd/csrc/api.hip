// Host-side plumbing shared by the C ABI entry points: thread-local error text, launch checks.
#include <stdarg.h>
#include <stdio.h>

#include "common.h"

namespace {
thread_local char g_err[512] = "";
}

namespace dsa_host {

dsa_status fail(dsa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

dsa_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return DSA_OK;
}

}  // namespace dsa_host

extern "C" const char* dsa_last_error(void) { return g_err; }
extern "C" const char* dsa_version(void) { return "dsa-mi355x 0.1 (gfx950)"; }
