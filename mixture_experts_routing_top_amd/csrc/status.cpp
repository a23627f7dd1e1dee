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
    case MOE_ERR_UNSUPPORTED: return "unsupported by this library";
    case MOE_ERR_WORKSPACE: return "workspace or state too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_DEVICE_CHECK: return "the device check flagged invalid input";
    default: return "unknown status";
  }
}

extern "C" const char* moe_last_error(void) { return g_last_error; }

// The device-check word: wait for the stream, read the word, name its bits.
extern "C" int moe_check_device_error(const int32_t* check, int32_t* bits, void* stream) {
  using namespace moe;
  if (!check) return fail(MOE_ERR_INVALID_ARG, "moe_check_device_error: null check word");
  const hipStream_t s = as_stream(stream);
  int32_t word = 0;
  if (int rc = hip_status(hipMemcpyAsync(&word, check, sizeof(word), hipMemcpyDeviceToHost, s),
                          "moe_check_device_error readback"))
    return rc;
  if (int rc = hip_status(hipStreamSynchronize(s), "moe_check_device_error sync")) return rc;
  if (bits) *bits = word;
  if (word == 0) return MOE_OK;
  static const struct { int32_t bit; const char* what; } kNames[] = {
      {MOE_CHECK_LOGITS, "non-finite router logits"},
      {MOE_CHECK_INDEX, "expert index outside [0, E)"},
      {MOE_CHECK_DUPLICATE, "a token names one expert twice"},
      {MOE_CHECK_COUNTS, "counts differ from the routing"},
      {MOE_CHECK_REPLICAS, "negative replica count or copies beyond max_slots"},
      {MOE_CHECK_SLOTS, "invalid slot table"},
      {MOE_CHECK_ROWS, "inv_pos entry outside [0, M)"},
  };
  char msg[400];
  int n = snprintf(msg, sizeof(msg), "device check 0x%x:", static_cast<unsigned>(word));
  for (const auto& k : kNames)
    if ((word & k.bit) && n > 0 && n < static_cast<int>(sizeof(msg)))
      n += snprintf(msg + n, sizeof(msg) - n, " %s;", k.what);
  return fail(MOE_ERR_DEVICE_CHECK, "%s", msg);
}
