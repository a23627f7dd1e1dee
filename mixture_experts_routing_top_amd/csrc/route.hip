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
// Layout on gfx950: a group of G lanes (G a power of two, at most 16) owns one
// token; lane g holds J chunks of 4 consecutive logits, chunks g, g + G, ...
// (16-byte loads when the row allows it; G * 4 * J >= E, J > 1 only above
// E = 64).  k rounds of an arg-max over the group's lanes (DPP moves inside a
// 16-lane row), ordered by (logit desc, index asc), pick the experts; the
// winner's owner lane masks its entry.  HBM-bound: 4E bytes in, 8k bytes out per token.  With a check
// word, a NaN or infinite logit raises MOE_CHECK_LOGITS (the softmax routing
// of the pages is defined over finite logits).
#include <cfloat>

#include "common.h"

namespace {

__device__ __forceinline__ bool better(float v1, int i1, float v2, int i2) {
  return v1 > v2 || (v1 == v2 && i1 < i2);
}

// One step of the group arg-max (dpp_partner): after steps 1, 2, ... up to
// G / 2 every lane of an aligned group of G lanes holds the group's best
// (value, index).
template <int OFF>
__device__ __forceinline__ void argmax_step(float& bv, int& bi) {
  const float ov = __int_as_float(dpp_partner<OFF>(__float_as_int(bv)));
  const int oi = dpp_partner<OFF>(bi);
  if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
}

template <int G, int J>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits, int64_t T, int E, int k,
                                                    bool vec4, int32_t* __restrict__ topk_idx,
                                                    float* __restrict__ topk_w, int32_t* __restrict__ check) {
  constexpr int kTokPerBlock = 256 / G;
  constexpr int V = 4 * J;  // logits per lane
  const int g = threadIdx.x % G;
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTokPerBlock + threadIdx.x / G;
  const bool active = t < T;
  const float* row = logits + (active ? t : 0) * static_cast<int64_t>(E);
  // expert index of slot 4 j + c of this lane
  auto index_of = [&](int j, int c) { return 4 * (g + G * j) + c; };

  float v[V];
  unsigned taken = 0;  // bit s: slot s is chosen or holds no expert
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int base = index_of(j, 0);
    if (vec4 && base < E) {
      const float4 q = *reinterpret_cast<const float4*>(row + base);
      v[4 * j] = q.x; v[4 * j + 1] = q.y; v[4 * j + 2] = q.z; v[4 * j + 3] = q.w;
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c) v[4 * j + c] = (base + c < E) ? row[base + c] : -INFINITY;
    }
  }
  bool bad = false;
#pragma unroll
  for (int sl = 0; sl < V; ++sl) {
    if (index_of(sl / 4, sl % 4) >= E) taken |= 1u << sl;
    else bad |= active && !(fabsf(v[sl]) <= FLT_MAX);  // NaN or +-inf
    if (!(v[sl] == v[sl])) v[sl] = -INFINITY;  // NaN orders as -inf
  }
  if (check) raise_check(check, bad, MOE_CHECK_LOGITS);

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
      for (int sl = 0; sl < V; ++sl) {
        const int ix = index_of(sl / 4, sl % 4);
        if (!((taken >> sl) & 1u) && better(v[sl], ix, bv, bi)) { bv = v[sl]; bi = ix; }
      }
      static_assert(G <= 16, "a token's lanes lie in one DPP row");
      if constexpr (G >= 2) argmax_step<1>(bv, bi);
      if constexpr (G >= 4) argmax_step<2>(bv, bi);
      if constexpr (G >= 8) argmax_step<4>(bv, bi);
      if constexpr (G >= 16) argmax_step<8>(bv, bi);
      win_v[i] = bv;
      win_i[i] = bi;
      // the owner of expert bi: chunk bi / 4 = g + G j
      const int chunk = bi >> 2;
      if (chunk % G == g) taken |= 1u << (4 * (chunk / G) + (bi & 3));
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

template <int G, int J = 1>
void launch(const float* logits, int64_t T, int E, int k, bool vec4, int32_t* idx, float* w, int32_t* check,
            hipStream_t s) {
  const int64_t blocks = moe::ceil_div(T, 256 / G);
  route_kernel<G, J><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(logits, T, E, k, vec4, idx, w, check);
}

}  // namespace

extern "C" int moe_route(const float* logits, int64_t T, int E, int k, int32_t* topk_idx, float* topk_w,
                         int32_t* check, void* stream) {
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
  if (lanes <= 1) launch<1>(logits, T, E, k, vec4, topk_idx, topk_w, check, s);
  else if (lanes <= 2) launch<2>(logits, T, E, k, vec4, topk_idx, topk_w, check, s);
  else if (lanes <= 4) launch<4>(logits, T, E, k, vec4, topk_idx, topk_w, check, s);
  else if (lanes <= 8) launch<8>(logits, T, E, k, vec4, topk_idx, topk_w, check, s);
  else if (lanes <= 16) launch<16>(logits, T, E, k, vec4, topk_idx, topk_w, check, s);
  else if (lanes <= 32) launch<16, 2>(logits, T, E, k, vec4, topk_idx, topk_w, check, s);
  else if (lanes <= 48) launch<16, 3>(logits, T, E, k, vec4, topk_idx, topk_w, check, s);
  else launch<16, 4>(logits, T, E, k, vec4, topk_idx, topk_w, check, s);
  return hip_status(hipGetLastError(), "moe_route launch");
}
