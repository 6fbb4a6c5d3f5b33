// Host-side plumbing shared by the C ABI entry points: thread-local error text, launch checks.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

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

bool debug_poison() {
  const char* e = getenv("DSA_DEBUG_POISON");
  return e && e[0] == '1';
}

}  // namespace dsa_host

namespace dsa {
__global__ void __launch_bounds__(256) fill_ones(uint32_t* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0xFFFFFFFFu;
}
}  // namespace dsa

namespace dsa_host {
void poison_fill(void* p, size_t bytes, hipStream_t s) {
  const size_t n = bytes / 4;
  if (!p || n == 0) return;
  const unsigned blocks = (unsigned)(n / 256 + 1 < 1024 ? n / 256 + 1 : 1024);
  hipLaunchKernelGGL(dsa::fill_ones, dim3(blocks), dim3(256), 0, s, (uint32_t*)p, n);
}
}  // namespace dsa_host

extern "C" const char* dsa_last_error(void) { return g_err; }
extern "C" const char* dsa_version(void) { return "dsa-mi355x 0.1 (gfx950)"; }
