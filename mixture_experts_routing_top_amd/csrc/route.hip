// moe_route: top-k softmax gate with renormalised weights.
//
// Source: the naive top-k gate of "PopFetcher: Towards Accelerated
// Mixture-of-Experts Training Via Popularity Based Expert-Wise Prefetch (ATC
// 2025)" (observations, trade-offs) and the softmax routing named in "Fast MoE
// Inference via Predictive Prefetching and Expert Replication" (problem
// statement): softmax over the E router logits, keep the k largest, renormalise
// the kept probabilities.  Because the renormalisation divides by the kept
// mass, w_i = exp(l_i - m) / sum_j exp(l_j - m) over the kept logits only: the
// full softmax denominator cancels and is never formed.
//
// Layout on gfx950: a group of G lanes (G a power of two, G * 4 >= E) owns one
// token; each lane holds 4 consecutive logits (one 16-byte load when the row
// allows it).  k rounds of a butterfly arg-max over the group's lanes, ordered
// by (logit desc, index asc), pick the experts; the winner's owner lane masks
// its entry.  HBM-bound: 4E bytes in, 8k bytes out per token.
#include <cfloat>

#include "common.h"

namespace {

__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

template <int G>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int64_t T, int E, int k,
                                                    bool vec4, int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w) {
  constexpr int kTokPerBlock = 256 / G;
  const int g = threadIdx.x % G;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokPerBlock + threadIdx.x / G;
  const bool active = t < T;
  const float* row = logits + (active ? t : 0) * static_cast<int64_t>(E);
  const int base = 4 * g;

  float v[4];
  unsigned taken = 0;  // bit c: entry c is chosen or does not exist
  if (vec4 && base < E) {
    const float4 q = *reinterpret_cast<const float4*>(row + base);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = (base + c < E) ? row[base + c] : -INFINITY;
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if (base + c >= E) taken |= 1u << c;
    if (!(v[c] == v[c])) v[c] = -INFINITY;  // NaN orders as -inf
  }

  float win_v[moe::kMaxTopK];
  int win_i[moe::kMaxTopK];
#pragma unroll
  for (int i = 0; i < moe::kMaxTopK; ++i) {
    win_v[i] = -INFINITY;
    win_i[i] = 0;
    if (i < k) {
      float bv = -INFINITY;
      int bi = INT32_MAX;
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (!((taken >> c) & 1u) && better(v[c], base + c, bv, bi)) { bv = v[c]; bi = base + c; }
#pragma unroll
      for (int off = 1; off < G; off <<= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      win_v[i] = bv;
      win_i[i] = bi;
      if ((bi >> 2) == g) taken |= 1u << (bi & 3);
    }
  }

  if (!active) return;
  const float m = win_v[0];
  float e[moe::kMaxTopK];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < moe::kMaxTopK; ++i) {
    e[i] = (i < k) ? expf(win_v[i] - m) : 0.f;
    s += e[i];
  }
#pragma unroll
  for (int i = 0; i < moe::kMaxTopK; ++i) {
    if (i < k && (i % G) == g) {
      topk_idx[t * k + i] = win_i[i];
      topk_w[t * k + i] = e[i] / s;
    }
  }
}

template <int G>
void launch(const float* logits, int64_t T, int E, int k, bool vec4, int32_t* idx, float* w, hipStream_t s) {
  const int64_t blocks = moe::ceil_div(T, 256 / G);
  route_kernel<G><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(logits, T, E, k, vec4, idx, w);
}

}  // namespace

extern "C" int moe_route(const float* logits, int64_t T, int E, int k, int32_t* topk_idx, float* topk_w,
                         void* stream) {
  using namespace moe;
  if (E < 1 || E > kMaxExperts) return fail(E < 1 ? MOE_ERR_INVALID_ARG : MOE_ERR_UNSUPPORTED,
                                            "moe_route: E=%d outside [1, %d]", E, kMaxExperts);
  if (k < 1 || k > E || k > kMaxTopK) return fail(MOE_ERR_INVALID_ARG, "moe_route: k=%d outside [1, min(E, 8)]", k);
  if (T < 0 || T * k >= (int64_t(1) << 31)) return fail(MOE_ERR_INVALID_ARG, "moe_route: T=%lld out of range", (long long)T);
  if (T == 0) return MOE_OK;
  if (!logits || !topk_idx || !topk_w) return fail(MOE_ERR_INVALID_ARG, "moe_route: null pointer");
  const bool vec4 = (E % 4 == 0) && aligned16(logits);
  const hipStream_t s = as_stream(stream);
  const int lanes = static_cast<int>(ceil_div(E, 4));
  if (lanes <= 1) launch<1>(logits, T, E, k, vec4, topk_idx, topk_w, s);
  else if (lanes <= 2) launch<2>(logits, T, E, k, vec4, topk_idx, topk_w, s);
  else if (lanes <= 4) launch<4>(logits, T, E, k, vec4, topk_idx, topk_w, s);
  else if (lanes <= 8) launch<8>(logits, T, E, k, vec4, topk_idx, topk_w, s);
  else if (lanes <= 16) launch<16>(logits, T, E, k, vec4, topk_idx, topk_w, s);
  else if (lanes <= 32) launch<32>(logits, T, E, k, vec4, topk_idx, topk_w, s);
  else launch<64>(logits, T, E, k, vec4, topk_idx, topk_w, s);
  return hip_status(hipGetLastError(), "moe_route launch");
}
