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

// Upper bounds of the library.
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 8;

}  // namespace moe

// ---- device helpers ------------------------------------------------------
// Device check: OR `bits` into the caller's check word once per wave whose
// lanes flag anything (a vector atomic from the first flagging lane).  Every
// lane of the wave must call it (the ballot is wave-wide).
__device__ __forceinline__ void raise_check(int32_t* check, bool flagged, int32_t bits) {
  const uint64_t m = __ballot(flagged);
  if (m != 0 && (__lane_id() == static_cast<unsigned>(__ffsll(static_cast<unsigned long long>(m)) - 1)))
    atomicOr(check, bits);
}

// The value of the lane OFF away in an all-reduce pairing inside a 16-lane
// row, by a DPP move (a VALU operand modifier, no LDS round trip):
// quad_perm(1,0,3,2) for OFF = 1, quad_perm(2,3,0,1) for 2, row_half_mirror
// (i <-> 7 - i in eight lanes) for 4, row_mirror (i <-> 15 - i in sixteen)
// for 8.  Combining with an associative, commutative operation after steps 1,
// 2, ... up to G / 2 leaves every lane of an aligned group of G lanes with the
// group's result.
template <int OFF>
__device__ __forceinline__ int dpp_partner(int x) {
  static_assert(OFF == 1 || OFF == 2 || OFF == 4 || OFF == 8, "pairings inside one DPP row");
  if constexpr (OFF == 1) return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);
  else if constexpr (OFF == 2) return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);
  else if constexpr (OFF == 4) return __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);
  else return __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
