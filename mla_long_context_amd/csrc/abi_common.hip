// Thread-local error reporting for the C ABI.
#include <stdarg.h>
#include <stdio.h>

#include <atomic>

#include "mla_internal.h"

namespace {
thread_local char g_err[512] = {0};
}

void mla_set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

void mla_clear_error() { g_err[0] = 0; }

void mla_begin_call() {
  g_err[0] = 0;
  // An error left in the runtime's per-thread slot by an earlier, unrelated
  // call (another library, a failed launch of the caller's own) is not this
  // call's: it is discarded here, so that the check after this call's
  // launches reports only what they did.
  (void)hipGetLastError();
}

int mla_check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    mla_set_error("%s: launch failed: %s", what, hipGetErrorString(e));
    return MLA_ERR_LAUNCH;
  }
  return MLA_OK;
}

int mla_num_cus() {
  // per-device cache of the compute-unit count (persistent kernels size
  // their grids by it); 0 until first asked on that device. Entries are
  // atomics: threads that race on the first query store the same value.
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (dev < 0 || dev >= 64) return 0;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 0;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

extern "C" const char* mla_last_error(void) { return g_err; }

extern "C" int mla_abi_version(void) { return 2; }
