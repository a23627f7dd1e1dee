// Greedy, capacity-bounded replica plan over E <= 256 experts, run by one wave.
//
// Sources: the MoE-GPS blog, section 2.1 (duplicate_experts gives an expert
// whose load exceeds the target extra copies); "Fast MoE Inference via
// Predictive Prefetching and Expert Replication", contribution 3 (the number
// of replicas is bounded by a memory budget); PopFetcher wiki, method (the
// budget is filled greedily by popularity).
//
// The budget is handed out one copy at a time to the expert with the largest
// per-copy load n_e / (r_e + 1) among those still above the mean per copy
// (n_e * E > total * (r_e + 1)); equal per-copy loads go to the lower index;
// the plan stops when no expert qualifies.  All comparisons are exact int64
// cross-multiplications.  Lane l holds experts l, l+64, l+128, l+192.
#pragma once

#include "common.h"

namespace moe {

// (n_a, r_a, a) has a larger per-copy load than (n_b, r_b, b); ties -> lower index.
__device__ __forceinline__ bool heavier(int64_t na, int ra, int a, int64_t nb, int rb, int b) {
  if (b < 0) return a >= 0;
  if (a < 0) return false;
  const int64_t l = na * (rb + 1), r = nb * (ra + 1);
  return l > r || (l == r && a < b);
}

// Called by all 64 lanes of one wave; n[j] is expert lane + 64 j's load (0
// past E), total the sum the target is taken from; r[j] receives the copies.
__device__ inline void plan_replicas_wave(const int64_t (&n)[4], int E, int64_t total, int budget, int lane,
                                          int (&r)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = 0;
  for (int step = 0; step < budget; ++step) {
    int64_t bn = 0;
    int br = 0, be = -1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = lane + 64 * j;
      const bool above = e < E && n[j] * E > total * (r[j] + 1);
      if (above && heavier(n[j], r[j], e, bn, br, be)) { bn = n[j]; br = r[j]; be = e; }
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t on = __shfl_xor(bn, off);
      const int orr = __shfl_xor(br, off);
      const int oe = __shfl_xor(be, off);
      if (heavier(on, orr, oe, bn, br, be)) { bn = on; br = orr; be = oe; }
    }
    if (be < 0) break;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j == be) r[j] += 1;
  }
}

}  // namespace moe
