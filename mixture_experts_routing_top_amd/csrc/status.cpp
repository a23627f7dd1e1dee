// Status strings and the per-thread last-error message of the C ABI.
#include <cstdarg>
#include <cstdio>

#include "common.h"

namespace {
thread_local char g_last_error[512] = "";
}

namespace moe {

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int hip_status(hipError_t err, const char* what) {
  if (err == hipSuccess) return MOE_OK;
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(err));
}

}  // namespace moe

extern "C" const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported by this build";
    case MOE_ERR_WORKSPACE: return "workspace or state too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

extern "C" const char* moe_last_error(void) { return g_last_error; }
