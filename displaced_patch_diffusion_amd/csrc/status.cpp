// Status strings and the thread-local last-error record of libdp.
#include <stdarg.h>
#include <stdio.h>

#include "dp_internal.h"

namespace {
thread_local char g_last_error[512] = "";
}

namespace dp {

dp_status fail(dp_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_last_error[0] = '\0'; }

dp_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(DP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return DP_OK;
}

}  // namespace dp

DP_API const char* dp_status_string(dp_status s) {
  switch (s) {
    case DP_OK: return "ok";
    case DP_ERR_INVALID_ARG: return "invalid argument";
    case DP_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case DP_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

DP_API const char* dp_last_error(void) { return g_last_error; }
