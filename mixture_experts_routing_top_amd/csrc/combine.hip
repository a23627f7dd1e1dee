// moe_combine: weighted combine of the k expert outputs back to token order.
//
// Source: the LocalReduce that follows the expert computation in the EPS-MoE
// review, section 3 (memory-bound, overlappable): out[t] = sum_i w[t,i] *
// y_perm[inv_pos[t,i]], with the renormalised gate weights of the top-k gate.
//
// Four 16-byte chunks of one output row per thread (strided so a wave's
// accesses stay contiguous): k gathers each from the expert-ordered rows, fp32
// FMAs in slot order, one rounding to the dtype, 16-byte stores.  HBM-bound:
// (k + 1) * H * s bytes per token.  With a check word, an inv_pos entry
// outside [0, M) (skipped) raises MOE_CHECK_ROWS.
#include "common.h"

namespace {

constexpr int kChunksPerThread = 4;

// Thread (t, c0) handles chunks c0, c0 + stride, ... of token t's row: the
// token's k row indices and weights are read once, and its k x 4 gathers are
// independent loads in flight together.
template <bool kBf16>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ y, int64_t M,
                                                      const int32_t* __restrict__ inv_pos,
                                                      const float* __restrict__ w, int64_t T, int k, int chunks,
                                                      uint4* __restrict__ out, int32_t* __restrict__ check) {
  const int groups = (chunks + kChunksPerThread - 1) / kChunksPerThread;  // threads per token
  const int64_t g = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (check) {  // one thread per token looks at its k rows (before any lane leaves)
    bool bad = false;
    if (g < T * groups && g % groups == 0)
      for (int i = 0; i < k; ++i) {
        const int32_t r = inv_pos[(g / groups) * k + i];
        bad |= r < 0 || r >= M;
      }
    raise_check(check, bad, MOE_CHECK_ROWS);
  }
  if (g >= T * groups) return;
  const int64_t t = g / groups;
  const int c0 = static_cast<int>(g - t * groups);
  constexpr int V = kBf16 ? 8 : 4;
  float acc[kChunksPerThread][V];
#pragma unroll
  for (int u = 0; u < kChunksPerThread; ++u)
#pragma unroll
    for (int j = 0; j < V; ++j) acc[u][j] = 0.f;
  for (int i = 0; i < k; ++i) {
    const int32_t r = inv_pos[t * k + i];
    if (r < 0 || r >= M) continue;
    const float wi = w[t * k + i];
    const uint4* row = y + static_cast<int64_t>(r) * chunks;
    uint4 q[kChunksPerThread];
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
      const int c = c0 + u * groups;
      q[u] = c < chunks ? row[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
      const uint32_t v[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
      if constexpr (kBf16) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[u][2 * j] = fmaf(wi, bf16_bits_to_f32(v[j] & 0xffffu), acc[u][2 * j]);
          acc[u][2 * j + 1] = fmaf(wi, bf16_bits_to_f32(v[j] >> 16), acc[u][2 * j + 1]);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[u][j] = fmaf(wi, __uint_as_float(v[j]), acc[u][j]);
      }
    }
  }
  uint4* orow = out + t * chunks;
#pragma unroll
  for (int u = 0; u < kChunksPerThread; ++u) {
    const int c = c0 + u * groups;
    if (c >= chunks) continue;
    uint4 o;
    if constexpr (kBf16) {
      o.x = f32_to_bf16_bits(acc[u][0]) | (f32_to_bf16_bits(acc[u][1]) << 16);
      o.y = f32_to_bf16_bits(acc[u][2]) | (f32_to_bf16_bits(acc[u][3]) << 16);
      o.z = f32_to_bf16_bits(acc[u][4]) | (f32_to_bf16_bits(acc[u][5]) << 16);
      o.w = f32_to_bf16_bits(acc[u][6]) | (f32_to_bf16_bits(acc[u][7]) << 16);
    } else {
      o.x = __float_as_uint(acc[u][0]);
      o.y = __float_as_uint(acc[u][1]);
      o.z = __float_as_uint(acc[u][2]);
      o.w = __float_as_uint(acc[u][3]);
    }
    orow[c] = o;
  }
}

}  // namespace

extern "C" int moe_combine(const void* y_perm, moe_dtype dt, int64_t M, const int32_t* inv_pos, const float* topk_w,
                           int64_t T, int k, int H, void* out, int32_t* check, void* stream) {
  using namespace moe;
  if (dt != MOE_F32 && dt != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "moe_combine: unknown dtype %d", (int)dt);
  if (k < 1 || k > kMaxTopK) return fail(MOE_ERR_INVALID_ARG, "moe_combine: k=%d outside [1, 8]", k);
  if (T < 0 || M < 0 || T * k >= (int64_t(1) << 31)) return fail(MOE_ERR_INVALID_ARG, "moe_combine: bad T or M");
  if (H < 1 || (static_cast<int64_t>(H) * elem_bytes(dt)) % 16 != 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_combine: H*sizeof(dtype) must be a positive multiple of 16 (H=%d)", H);
  if (T == 0) return MOE_OK;
  if (!inv_pos || !topk_w || !out || (M > 0 && !y_perm)) return fail(MOE_ERR_INVALID_ARG, "moe_combine: null pointer");
  if (!aligned16(out) || (y_perm && !aligned16(y_perm)))
    return fail(MOE_ERR_INVALID_ARG, "moe_combine: y_perm and out must be 16-byte aligned");
  const int chunks = static_cast<int>(static_cast<int64_t>(H) * elem_bytes(dt) / 16);
  const int64_t groups = ceil_div(chunks, kChunksPerThread);
  const unsigned blocks = static_cast<unsigned>(ceil_div(T * groups, 256));
  const hipStream_t s = as_stream(stream);
  if (dt == MOE_BF16)
    combine_kernel<true><<<blocks, 256, 0, s>>>(static_cast<const uint4*>(y_perm), M, inv_pos, topk_w, T, k, chunks,
                                               static_cast<uint4*>(out), check);
  else
    combine_kernel<false><<<blocks, 256, 0, s>>>(static_cast<const uint4*>(y_perm), M, inv_pos, topk_w, T, k, chunks,
                                                static_cast<uint4*>(out), check);
  return hip_status(hipGetLastError(), "moe_combine launch");
}
