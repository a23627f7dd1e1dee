// moe_plan_replicas and moe_prediction_quality: replicas planned ahead of
// routing from a predicted expert distribution, and how well a prediction and
// a plan matched the routing that followed.
//
// Sources: "PopFetcher: Towards Accelerated Mixture-of-Experts Training Via
// Popularity Based Expert-Wise Prefetch (ATC 2025)", method (Eq.(3) predicts
// the next layer's popularity before it runs, and the plan acts on it); "Fast
// MoE Inference via Predictive Prefetching and Expert Replication",
// contributions 2-3 (replicas placed from predicted activity, within a budget;
// prediction accuracy and load balance as the measures); the MoE-GPS blog,
// section 2.1 (copies sized so per-copy load nears the mean).
//
// Both are single-block kernels over E <= 256 experts (microseconds).  The
// plan rounds p_hat * total to integer rows (halves to even) and runs the same
// greedy planner as moe_stats.  The quality kernel ranks experts in parallel
// and takes its sums in expert order in one thread, in double with explicitly
// rounded operations, so its results do not depend on scheduling.
#include <cmath>

#include "common.h"
#include "replica_plan.h"

namespace {

__global__ __launch_bounds__(64) void plan_kernel(const float* __restrict__ pred, int E, int64_t total, int budget,
                                                  int32_t* __restrict__ pred_counts,
                                                  int32_t* __restrict__ replicas) {
  const int lane = threadIdx.x;
  int64_t n[4];
  int64_t part = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    int32_t c = 0;
    if (e < E) {
      const double v = __dmul_rn(static_cast<double>(pred[e]), static_cast<double>(total));
      if (!(v > 0.0)) c = 0;
      else if (v >= 2147483647.0) c = 2147483647;
      else c = static_cast<int32_t>(rint(v));  // nearest, halves to even
      if (pred_counts) pred_counts[e] = c;
    }
    n[j] = c;
    part += c;
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) part += __shfl_xor(part, off);
  int r[4];
  moe::plan_replicas_wave(n, E, part, budget, lane, r);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (lane + 64 * j < E) replicas[lane + 64 * j] = r[j];
}

// NaN ranks as -inf
__device__ __forceinline__ double rank_value(double v) { return v != v ? -INFINITY : v; }

// extra copies of expert e, clamped to [0, 4096]
__device__ __forceinline__ int64_t copies_of(const int32_t* replicas, int e) {
  return 1 + (replicas ? min(max(replicas[e], 0), 4096) : 0);
}

__global__ __launch_bounds__(256) void quality_kernel(const float* __restrict__ pred,
                                                      const int32_t* __restrict__ counts, int E,
                                                      const int32_t* __restrict__ replicas, int top_n,
                                                      float* __restrict__ out) {
  __shared__ int hits;
  const int tid = threadIdx.x;
  const int n = min(top_n, E);
  if (tid == 0) hits = 0;
  __syncthreads();
  // expert e is in a top-n set iff fewer than n experts rank above it
  // (value descending, then index ascending)
  if (tid < E) {
    const double pv = rank_value(static_cast<double>(pred[tid]));
    const int32_t cv = counts[tid];
    int above_p = 0, above_c = 0;
    for (int x = 0; x < E; ++x) {
      const double px = rank_value(static_cast<double>(pred[x]));
      const int32_t cx = counts[x];
      above_p += (px > pv || (px == pv && x < tid)) ? 1 : 0;
      above_c += (cx > cv || (cx == cv && x < tid)) ? 1 : 0;
    }
    if (above_p < n && above_c < n) atomicAdd(&hits, 1);
  }
  __syncthreads();
  if (tid != 0) return;
  double S = 0.0;
  int64_t A = 0;
  for (int e = 0; e < E; ++e) {
    S = __dadd_rn(S, static_cast<double>(pred[e]));
    A += counts[e];
  }
  double tv = 1.0;
  if (S > 0.0 && A > 0) {
    double acc = 0.0;
    for (int e = 0; e < E; ++e)
      acc = __dadd_rn(acc, fabs(__dsub_rn(__ddiv_rn(static_cast<double>(pred[e]), S),
                                          __ddiv_rn(static_cast<double>(counts[e]), static_cast<double>(A)))));
    tv = __dmul_rn(0.5, acc);
  }
  int64_t slots = 0, mx = 0;
  for (int e = 0; e < E; ++e) slots += copies_of(replicas, e);
  const double mean = __ddiv_rn(static_cast<double>(A), static_cast<double>(slots));
  double var = 0.0;
  for (int e = 0; e < E; ++e) {
    const int64_t copies = copies_of(replicas, e);
    const int64_t ne = counts[e];
    for (int64_t rho = 0; rho < copies; ++rho) {
      const int64_t load = ((rho + 1) * ne) / copies - (rho * ne) / copies;
      const double d = __dsub_rn(static_cast<double>(load), mean);
      var = __dadd_rn(var, __dmul_rn(d, d));
      mx = max(mx, load);
    }
  }
  out[0] = static_cast<float>(tv);
  out[1] = static_cast<float>(__ddiv_rn(static_cast<double>(hits), static_cast<double>(n)));
  out[2] = static_cast<float>(__dsqrt_rn(__ddiv_rn(var, static_cast<double>(slots))));
  out[3] = A > 0 ? static_cast<float>(__ddiv_rn(static_cast<double>(mx), mean)) : 0.0f;
}

}  // namespace

extern "C" int moe_plan_replicas(const float* pred, int E, int64_t total, int replica_budget, int32_t* pred_counts,
                                 int32_t* replicas, void* stream) {
  using namespace moe;
  if (E < 1 || E > kMaxExperts)
    return fail(E < 1 ? MOE_ERR_INVALID_ARG : MOE_ERR_UNSUPPORTED, "moe_plan_replicas: E=%d outside [1, %d]", E,
                kMaxExperts);
  if (total < 0 || total >= (int64_t(1) << 31))
    return fail(MOE_ERR_INVALID_ARG, "moe_plan_replicas: total=%lld outside [0, 2^31)", (long long)total);
  if (replica_budget < 0 || replica_budget > 4096)
    return fail(MOE_ERR_INVALID_ARG, "moe_plan_replicas: replica_budget=%d outside [0, 4096]", replica_budget);
  if (!pred || !replicas) return fail(MOE_ERR_INVALID_ARG, "moe_plan_replicas: null pointer");
  plan_kernel<<<1, 64, 0, as_stream(stream)>>>(pred, E, total, replica_budget, pred_counts, replicas);
  return hip_status(hipGetLastError(), "moe_plan_replicas launch");
}

extern "C" int moe_prediction_quality(const float* pred, const int32_t* counts, int E, const int32_t* replicas,
                                      int top_n, float* out, void* stream) {
  using namespace moe;
  if (E < 1 || E > kMaxExperts)
    return fail(E < 1 ? MOE_ERR_INVALID_ARG : MOE_ERR_UNSUPPORTED, "moe_prediction_quality: E=%d outside [1, %d]",
                E, kMaxExperts);
  if (top_n < 1) return fail(MOE_ERR_INVALID_ARG, "moe_prediction_quality: top_n=%d must be >= 1", top_n);
  if (!pred || !counts || !out) return fail(MOE_ERR_INVALID_ARG, "moe_prediction_quality: null pointer");
  quality_kernel<<<1, 256, 0, as_stream(stream)>>>(pred, counts, E, replicas, top_n, out);
  return hip_status(hipGetLastError(), "moe_prediction_quality launch");
}
