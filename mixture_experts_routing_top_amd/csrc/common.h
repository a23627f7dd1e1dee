// Internal helpers shared by the HIP translation units of libmoe_mi355x.so.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "moe.h"

namespace moe {

// Record a message for moe_last_error() and return `status`.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Map a HIP error (typically from a launch) to MOE_ERR_HIP with its text.
int hip_status(hipError_t err, const char* what);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int elem_bytes(moe_dtype dt) { return dt == MOE_BF16 ? 2 : 4; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Upper bounds of this build.
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 8;

}  // namespace moe

// ---- device helpers ------------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
