// Error reporting and version entry points of the C ABI.
#include <stdarg.h>
#include <stdio.h>

#include "common.h"

namespace {
thread_local char g_msg[512] = "";
}

namespace bqm {

bqm_status fail(bqm_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return s;
}

bqm_status ok() { return BQM_OK; }

bqm_status launch_status(const char *what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(BQM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return BQM_OK;
}

}  // namespace bqm

extern "C" int bqm_abi_version(void) { return BQM_ABI_VERSION; }

extern "C" const char *bqm_last_error(void) { return g_msg; }
