// moe_stats: sliding-window routing statistics and the replica plan.
//
// Sources: "PopFetcher: Towards Accelerated Mixture-of-Experts Training Via
// Popularity Based Expert-Wise Prefetch (ATC 2025)", method (Routing
// Information Collector over a sliding window of s iterations; Eq.(1) sequence
// popularity, Eq.(2) layer-to-layer conditional probability, Eq.(3) next-layer
// popularity) and observation 2 (adjacent-layer correlation); the MoE-GPS blog,
// section 2.1 (p_i = n_i / N with a sliding-window average; duplicate_experts
// for loads above target); "Fast MoE Inference via Predictive Prefetching and
// Expert Replication", contribution 3 (replica counts bounded by a budget).
//
// One launch (two above E = 64).  Every block histograms its token range
// into LDS (counts, and the k*k co-occurrence pairs with the previous layer),
// then merges the non-zero bins into a device accumulator with atomics.  The
// block that takes the last ticket moves the accumulator into the ring slot
// (zeroing it for the next call), sums the ring, and derives popularity, the
// conditional matrix, the prediction and the replica counts.  Above E = 64 the
// E*E work (the co-occurrence ring update, the conditional matrix) is too much
// for one block: a second launch spreads it over blocks of 2048 cells and of
// four rows, and the last of the row blocks (ticket) sums the prediction.  All counts are exact
// integers; the divisions are IEEE fp32 divisions of exact integers and the
// prediction is a double sum in expert order, so the results do not depend on
// the order in which blocks finish.  With a check word, indices outside [0, E)
// (skipped) raise MOE_CHECK_INDEX and a token naming one expert twice (counted
// as often as named) MOE_CHECK_DUPLICATE: the top-k gate picks k distinct
// experts.
#include "common.h"
#include "replica_plan.h"

namespace {

constexpr int kThreads = 256;
constexpr int kTokPerBlock = 512;
// One block's co-occurrence counts are at most 512 tokens x k^2 = 32768 per
// cell, so while recording, two 16-bit counters share one LDS word: E*E up to
// 32768 cells (E <= 181) stays in LDS.  Up to 65536 cells (E <= 256) four
// 8-bit counters share a word, in blocks of 255 tokens (stats_kernel<true>):
// a token whose k experts are distinct, and whose previous layer's are too,
// adds at most one to a cell; a token naming an expert twice adds into global
// memory instead.
constexpr int kLdsCooc = 128 * 128;  // LDS words for co-occurrence
constexpr int kTokPerBlock8 = 255;
constexpr int kSplitE = 64;          // above: the E*E work runs in pair_kernel

struct Layout {
  size_t cnt_ring, cooc_ring, cooc_sum, acc, acc_cooc, ticket, ps, pmat, ticket2, words;
};

Layout layout(int L, int E, int window) {
  Layout q{};
  size_t w = 0;
  auto take = [&](size_t n) { size_t at = w; w = moe::align_up(w + n, 64); return at; };
  q.cnt_ring = take(static_cast<size_t>(window) * L * E);
  q.cooc_ring = take(static_cast<size_t>(window) * (L - 1) * E * E);
  q.cooc_sum = take(static_cast<size_t>(L - 1) * E * E);  // running sum of each pair's ring
  q.acc = take(E);
  q.acc_cooc = take(L > 1 ? static_cast<size_t>(E) * E : 0);
  q.ticket = take(1);
  // E > kSplitE: p_seq and the conditional matrix handed to pair_kernel, and its ticket
  q.ps = take(E);
  q.pmat = take(L > 1 ? static_cast<size_t>(E) * E : 0);
  q.ticket2 = take(1);
  q.words = w;
  return q;
}

struct Args {
  int32_t* state;
  Layout lay;
  int L, E, window, layer, slot, k, budget;
  int64_t T;
  const int32_t* idx;
  const int32_t* prev;
  int32_t* counts;
  float* p_seq;
  float* cond;
  float* pred;
  int32_t* replicas;
  int32_t* check;
};

template <bool k8>
__global__ __launch_bounds__(kThreads) void stats_kernel(Args a) {
  __shared__ int32_t hist[moe::kMaxExperts];
  __shared__ int32_t cooc[kLdsCooc];   // packed 16-bit (k8: 8-bit) counters of one block
  __shared__ int32_t nw[moe::kMaxExperts];
  __shared__ int32_t rowsum[moe::kMaxExperts];
  __shared__ float ps[moe::kMaxExperts];
  __shared__ unsigned long long total;
  __shared__ int is_last;

  const int E = a.E, k = a.k, tid = threadIdx.x;
  const int EE = E * E;
  const bool do_cooc = a.idx && a.layer > 0;
  const bool lds_cooc = !k8 && EE <= 2 * kLdsCooc;  // recording in LDS (packed 16-bit)
  constexpr int kTPB = k8 ? kTokPerBlock8 : kTokPerBlock;
  int32_t* acc = a.state + a.lay.acc;
  int32_t* acc_cooc = a.state + a.lay.acc_cooc;
  unsigned* ticket = reinterpret_cast<unsigned*>(a.state + a.lay.ticket);

  if (a.idx) {
    for (int e = tid; e < E; e += kThreads) hist[e] = 0;
    if (do_cooc && lds_cooc)
      for (int q = tid; q < (EE + 1) / 2; q += kThreads) cooc[q] = 0;
    if (k8 && do_cooc)
      for (int q = tid; q < (EE + 3) / 4; q += kThreads) cooc[q] = 0;
    __syncthreads();
    const int64_t t0 = static_cast<int64_t>(blockIdx.x) * kTPB;
    const int64_t t1 = min(a.T, t0 + kTPB);
    bool bad_index = false, bad_dup = false;
    for (int64_t t = t0 + tid; t < t1; t += kThreads) {
      int cur[moe::kMaxTopK];
#pragma unroll
      for (int i = 0; i < moe::kMaxTopK; ++i) {
        cur[i] = -1;
        if (i < k) {
          const int e = a.idx[t * k + i];
          if (e >= 0 && e < E) { cur[i] = e; atomicAdd(&hist[e], 1); }
          else bad_index = true;
        }
      }
      if (a.check) {
#pragma unroll
        for (int i = 1; i < moe::kMaxTopK; ++i)
#pragma unroll
          for (int j = 0; j < i; ++j) bad_dup |= i < k && cur[i] >= 0 && cur[i] == cur[j];
      }
      if (k8 && do_cooc) {
        int prv[moe::kMaxTopK];
        bool dup = false;  // an expert named twice by this token or by its previous layer
#pragma unroll
        for (int i = 0; i < moe::kMaxTopK; ++i) {
          prv[i] = -1;
          if (i < k) {
            const int p = a.prev[t * k + i];
            if (p >= 0 && p < E) prv[i] = p;
            else bad_index = true;
          }
        }
#pragma unroll
        for (int i = 1; i < moe::kMaxTopK; ++i)
#pragma unroll
          for (int j = 0; j < i; ++j)
            dup |= i < k && ((cur[i] >= 0 && cur[i] == cur[j]) || (prv[i] >= 0 && prv[i] == prv[j]));
#pragma unroll
        for (int i = 0; i < moe::kMaxTopK; ++i) {
          if (i >= k) break;
          if (prv[i] < 0) continue;
#pragma unroll
          for (int j = 0; j < moe::kMaxTopK; ++j) {
            if (j < k && cur[j] >= 0) {
              const int q = prv[i] * E + cur[j];
              if (!dup) atomicAdd(reinterpret_cast<unsigned*>(&cooc[q >> 2]), 1u << (8 * (q & 3)));
              else atomicAdd(&acc_cooc[q], 1);
            }
          }
        }
      } else if (do_cooc) {
#pragma unroll
        for (int i = 0; i < moe::kMaxTopK; ++i) {
          if (i >= k) break;
          const int p = a.prev[t * k + i];
          if (p < 0 || p >= E) {
            bad_index = true;
            continue;
          }
#pragma unroll
          for (int j = 0; j < moe::kMaxTopK; ++j) {
            if (j < k && cur[j] >= 0) {
              const int q = p * E + cur[j];
              if (lds_cooc) atomicAdd(reinterpret_cast<unsigned*>(&cooc[q >> 1]), 1u << (16 * (q & 1)));
              else atomicAdd(&acc_cooc[q], 1);
            }
          }
        }
      }
    }
    if (a.check) {
      raise_check(a.check, bad_index, MOE_CHECK_INDEX);
      raise_check(a.check, bad_dup, MOE_CHECK_DUPLICATE);
    }
    __syncthreads();
    for (int e = tid; e < E; e += kThreads)
      if (hist[e]) atomicAdd(&acc[e], hist[e]);
    if (do_cooc && lds_cooc)
      for (int q = tid; q < (EE + 1) / 2; q += kThreads) {
        const unsigned v = static_cast<unsigned>(cooc[q]);
        if (v & 0xffffu) atomicAdd(&acc_cooc[2 * q], static_cast<int32_t>(v & 0xffffu));
        if (v >> 16) atomicAdd(&acc_cooc[2 * q + 1], static_cast<int32_t>(v >> 16));
      }
    if (k8 && do_cooc)
      for (int q = tid; q < (EE + 3) / 4; q += kThreads) {
        const unsigned v = static_cast<unsigned>(cooc[q]);
#pragma unroll
        for (int b = 0; b < 4; ++b)
          if ((v >> (8 * b)) & 0xffu) atomicAdd(&acc_cooc[4 * q + b], static_cast<int32_t>((v >> (8 * b)) & 0xffu));
      }
    __threadfence();
    __syncthreads();
    if (tid == 0) is_last = (atomicAdd(ticket, 1u) == gridDim.x - 1);
    __syncthreads();
    if (!is_last) return;
    __threadfence();
  }

  // ---- finalize: one block ------------------------------------------------
  // Its global reads and writes are independent of one another (the ring
  // slot's new counts are added from registers, and the conditional matrix
  // reads the pair (layer, layer + 1), not the pair updated here), so they are
  // issued together and no fence is needed before the kernel ends.
  const int L = a.L, layer = a.layer, slot = a.slot, window = a.window;
  int32_t* cnt_ring = a.state + a.lay.cnt_ring;
  int32_t* cooc_ring = a.state + a.lay.cooc_ring;
  if (tid == 0) total = 0;
  __syncthreads();
  // Eq.(1): windowed popularity of this layer.  With this iteration's routing
  // the accumulator (zeroed for the next call) replaces the ring slot and the
  // window sum takes it from registers; the other slots come from the ring.
  for (int e = tid; e < E; e += kThreads) {
    const int32_t c = a.idx ? atomicExch(&acc[e], 0) : 0;
    int32_t s = 0;
    // unrolled so the window's loads are in flight together (exact integer sum)
#pragma unroll 8
    for (int w = 0; w < window; ++w)
      if (!a.idx || w != slot) s += cnt_ring[(static_cast<size_t>(w) * L + layer) * E + e];
    if (a.idx) {
      cnt_ring[(static_cast<size_t>(slot) * L + layer) * E + e] = c;
      hist[e] = c;
      if (a.counts) a.counts[e] = c;
      s += c;
    }
    nw[e] = s;
    atomicAdd(&total, static_cast<unsigned long long>(s));
  }
  const bool split = E > kSplitE;
  if (do_cooc && !split) {
    // the pair's ring slot is replaced and its running window sum updated by
    // the difference (exact integers: the sum over the ring, one load per cell)
    int32_t* cdst = cooc_ring + (static_cast<size_t>(slot) * (L - 1) + (layer - 1)) * EE;
    int32_t* csum = a.state + a.lay.cooc_sum + static_cast<size_t>(layer - 1) * EE;
    // eight cells per thread per round, every load and exchange issued before
    // the stores
    constexpr int U = 8;
    for (int q0 = tid; q0 < EE; q0 += U * kThreads) {
      int32_t old[U], sum[U], c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int q = q0 + u * kThreads;
        old[u] = q < EE ? cdst[q] : 0;
        sum[u] = q < EE ? csum[q] : 0;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int q = q0 + u * kThreads;
        c[u] = q < EE ? atomicExch(&acc_cooc[q], 0) : 0;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int q = q0 + u * kThreads;
        if (q < EE) {
          csum[q] = sum[u] + c[u] - old[u];
          cdst[q] = c[u];
        }
      }
    }
  }
  __syncthreads();
  const unsigned long long tot = total;
  for (int e = tid; e < E; e += kThreads) {
    const float p = tot ? __fdiv_rn(static_cast<float>(nw[e]), static_cast<float>(tot)) : 0.f;
    ps[e] = p;
    if (a.p_seq) a.p_seq[e] = p;
    if (split) reinterpret_cast<float*>(a.state + a.lay.ps)[e] = p;
  }

  // Eq.(2)-(3): conditional matrix of pair (layer, layer+1) and the prediction.
  // Up to E = 128 the window sums are read once and the matrix is kept in the
  // (now unused) co-occurrence LDS for the prediction's column sums; above, the
  // window sums are read from memory where needed.
  if (!split && layer + 1 < L && (a.cond || a.pred)) {
    const int32_t* win = a.state + a.lay.cooc_sum + static_cast<size_t>(layer) * EE;  // window sums
    for (int e = tid; e < E; e += kThreads) rowsum[e] = 0;
    __syncthreads();
    auto ratio = [&](int32_t c, int q) {
      const int32_t r = rowsum[q / E];
      return r ? __fdiv_rn(static_cast<float>(c), static_cast<float>(r)) : 0.f;
    };
    if (EE <= kLdsCooc) {
      for (int q = tid; q < EE; q += kThreads) {
        const int32_t c = win[q];
        cooc[q] = c;
        if (c) atomicAdd(&rowsum[q / E], c);
      }
      __syncthreads();
      for (int q = tid; q < EE; q += kThreads) {
        const float pq = ratio(cooc[q], q);
        if (a.cond) a.cond[q] = pq;
        cooc[q] = __float_as_int(pq);
      }
      __syncthreads();
      if (a.pred)
        for (int b = tid; b < E; b += kThreads) {
          double s = 0.0;
#pragma unroll 8
          for (int x = 0; x < E; ++x)
            s += static_cast<double>(ps[x]) * static_cast<double>(__int_as_float(cooc[x * E + b]));
          a.pred[b] = static_cast<float>(s);
        }
    } else {
      for (int q = tid; q < EE; q += kThreads) {
        const int32_t c = win[q];
        if (c) atomicAdd(&rowsum[q / E], c);
      }
      __syncthreads();
      if (a.cond)
        for (int q = tid; q < EE; q += kThreads) a.cond[q] = ratio(win[q], q);
      if (a.pred)
        for (int b = tid; b < E; b += kThreads) {
          double s = 0.0;
#pragma unroll 8
          for (int x = 0; x < E; ++x)
            s += static_cast<double>(ps[x]) * static_cast<double>(ratio(win[x * E + b], x * E + b));
          a.pred[b] = static_cast<float>(s);
        }
    }
  }

  // Replica plan from this iteration's counts (wave 0: 64 lanes x 4 experts).
  if (a.idx && a.replicas && tid < 64) {
    int64_t n[4];
    int r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) n[j] = tid + 64 * j < E ? hist[tid + 64 * j] : 0;
    moe::plan_replicas_wave(n, E, a.T * static_cast<int64_t>(k), a.budget, tid, r);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (tid + 64 * j < E) a.replicas[tid + 64 * j] = r[j];
  }
  if (a.idx && tid == 0) atomicExch(ticket, 0u);
}

// The E*E part of the finalize for E > kSplitE, after stats_kernel on the
// same stream: blocks [0, n_ring) replace pair (layer-1, layer)'s ring slot
// with the accumulator and update its running window sum (2048 cells each,
// eight per thread in flight); the row blocks after them take four rows of
// pair (layer, layer+1) each, one wave per row: the row's window sums, their
// exact integer row sum (a wave reduction) and the row-normalised
// probabilities, into cond and into the state for the prediction.  The last
// row block (ticket) sums the prediction in expert order from p_seq, which
// stats_kernel left in the state.  The same integers, fp32 divisions and
// double sums as the one-block finalize.
__global__ __launch_bounds__(kThreads) void pair_kernel(Args a, int n_ring, int n_rows) {
  __shared__ int is_last;
  const int E = a.E, EE = E * E, tid = threadIdx.x, L = a.L, layer = a.layer;
  if (static_cast<int>(blockIdx.x) < n_ring) {
    int32_t* cdst = a.state + a.lay.cooc_ring + (static_cast<size_t>(a.slot) * (L - 1) + (layer - 1)) * EE;
    int32_t* csum = a.state + a.lay.cooc_sum + static_cast<size_t>(layer - 1) * EE;
    int32_t* acc_cooc = a.state + a.lay.acc_cooc;
    constexpr int U = 8;
    const int q0 = blockIdx.x * (U * kThreads) + tid;
    int32_t old[U], sum[U], c[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = q0 + u * kThreads;
      old[u] = q < EE ? cdst[q] : 0;
      sum[u] = q < EE ? csum[q] : 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = q0 + u * kThreads;
      c[u] = q < EE ? atomicExch(&acc_cooc[q], 0) : 0;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int q = q0 + u * kThreads;
      if (q < EE) {
        csum[q] = sum[u] + c[u] - old[u];
        cdst[q] = c[u];
      }
    }
    return;
  }
  const int32_t* win = a.state + a.lay.cooc_sum + static_cast<size_t>(layer) * EE;  // window sums
  float* pmat = reinterpret_cast<float*>(a.state + a.lay.pmat);
  const int lane = tid & 63;
  const int x = (static_cast<int>(blockIdx.x) - n_ring) * (kThreads / 64) + (tid >> 6);
  if (x < E) {
    int32_t c[4];
    int32_t rs = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = lane + 64 * j;
      c[j] = b < E ? win[static_cast<size_t>(x) * E + b] : 0;
      rs += c[j];
    }
    for (int off = 32; off >= 1; off >>= 1) rs += __shfl_xor(rs, off);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int b = lane + 64 * j;
      if (b < E) {
        const float p = rs ? __fdiv_rn(static_cast<float>(c[j]), static_cast<float>(rs)) : 0.f;
        if (a.cond) a.cond[static_cast<size_t>(x) * E + b] = p;
        if (a.pred) pmat[static_cast<size_t>(x) * E + b] = p;
      }
    }
  }
  if (!a.pred) return;
  unsigned* ticket = reinterpret_cast<unsigned*>(a.state + a.lay.ticket2);
  __threadfence();
  __syncthreads();
  if (tid == 0) is_last = (atomicAdd(ticket, 1u) == static_cast<unsigned>(n_rows) - 1);
  __syncthreads();
  if (!is_last) return;
  __threadfence();
  const float* ps = reinterpret_cast<const float*>(a.state + a.lay.ps);
  for (int b = tid; b < E; b += kThreads) {
    double s = 0.0;
#pragma unroll 32
    for (int y = 0; y < E; ++y) s += static_cast<double>(ps[y]) * static_cast<double>(pmat[static_cast<size_t>(y) * E + b]);
    a.pred[b] = static_cast<float>(s);
  }
  if (tid == 0) atomicExch(ticket, 0u);
}

// Decayed-window popularity and the load-state check of one layer, read from
// the count ring (MoE-GPS blog, section 2.1: a decay factor on the sliding
// window; section 6.1: a load more than twice the history's standard
// deviation from its expectation; the load-prediction study: transient versus
// stable load states).  Thread e walks its expert's window youngest first:
//   D[e] = sum_age decay^age * n_e(age), weights by repeated multiplication;
//   anomalous when the window holds >= 2 earlier iterations and
//   (n_e(0) - mean)^2 > 4 * variance over those (else flagged: no history);
// p_decay = D / sum(D) in expert order; the layer is transient when more than a
// fifth of the experts are flagged.  Double arithmetic with explicitly rounded
// operations, in a fixed order, so the results do not depend on scheduling.
__global__ __launch_bounds__(kThreads) void load_state_kernel(const int32_t* __restrict__ cnt_ring, int L, int E,
                                                              int window, int layer, int slot0, int m,
                                                              double decay, float* __restrict__ p_decay,
                                                              int32_t* __restrict__ flags,
                                                              int32_t* __restrict__ summary) {
  __shared__ double D[moe::kMaxExperts];
  __shared__ double total;
  __shared__ int n_flagged;
  const int tid = threadIdx.x;
  if (tid == 0) n_flagged = 0;
  __syncthreads();
  auto at = [&](int age, int e) {
    int s = slot0 - age;
    if (s < 0) s += window;
    return static_cast<double>(cnt_ring[(static_cast<size_t>(s) * L + layer) * E + e]);
  };
  if (tid < E) {
    double d = 0.0, w = 1.0;
#pragma unroll 8
    for (int age = 0; age < m; ++age) {
      d = __dadd_rn(d, __dmul_rn(w, at(age, tid)));
      w = __dmul_rn(w, decay);
    }
    D[tid] = d;
    int f = 1;
    const int h = m - 1;
    if (h >= 2) {
      double sum = 0.0;
#pragma unroll 8
      for (int age = 1; age < m; ++age) sum = __dadd_rn(sum, at(age, tid));
      const double mu = __ddiv_rn(sum, static_cast<double>(h));
      double var = 0.0;
#pragma unroll 8
      for (int age = 1; age < m; ++age) {
        const double dd = __dsub_rn(at(age, tid), mu);
        var = __dadd_rn(var, __dmul_rn(dd, dd));
      }
      var = __ddiv_rn(var, static_cast<double>(h));
      const double d0 = __dsub_rn(at(0, tid), mu);
      f = __dmul_rn(d0, d0) > __dmul_rn(4.0, var) ? 1 : 0;
    }
    if (flags) flags[tid] = f;
    if (f) atomicAdd(&n_flagged, 1);
  }
  __syncthreads();
  if (tid == 0) {
    double t = 0.0;
    for (int e = 0; e < E; ++e) t = __dadd_rn(t, D[e]);
    total = t;
    if (summary) {
      summary[0] = n_flagged;
      summary[1] = 5 * n_flagged > E ? 1 : 0;
    }
  }
  __syncthreads();
  if (tid < E && p_decay) p_decay[tid] = total > 0.0 ? static_cast<float>(__ddiv_rn(D[tid], total)) : 0.0f;
}

__global__ void zero_words(int32_t* p, size_t n) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<size_t>(gridDim.x) * blockDim.x)
    p[i] = 0;
}

bool dims_ok(int L, int E, int window) {
  return L >= 1 && L <= 4096 && E >= 1 && E <= moe::kMaxExperts && window >= 1 && window <= 1024;
}

}  // namespace

extern "C" size_t moe_stats_state_bytes(int L, int E, int window) {
  if (!dims_ok(L, E, window)) return 0;
  return layout(L, E, window).words * sizeof(int32_t);
}

extern "C" int moe_stats_init(void* state, size_t state_bytes, int L, int E, int window, void* stream) {
  using namespace moe;
  if (!dims_ok(L, E, window)) return fail(MOE_ERR_INVALID_ARG, "moe_stats_init: bad L=%d E=%d window=%d", L, E, window);
  if (!state) return fail(MOE_ERR_INVALID_ARG, "moe_stats_init: null state");
  const size_t need = moe_stats_state_bytes(L, E, window);
  if (state_bytes < need) return fail(MOE_ERR_WORKSPACE, "moe_stats_init: state has %zu bytes, needs %zu", state_bytes, need);
  const size_t words = need / 4;
  const unsigned blocks = static_cast<unsigned>(std::min<size_t>(1024, ceil_div(words, 256)));
  zero_words<<<blocks, 256, 0, as_stream(stream)>>>(static_cast<int32_t*>(state), words);
  return hip_status(hipGetLastError(), "moe_stats_init launch");
}

extern "C" int moe_stats(void* state, size_t state_bytes, int L, int E, int window, int layer, int64_t iter,
                         const int32_t* topk_idx, const int32_t* prev_topk_idx, int64_t T, int k,
                         int32_t* counts, float* p_seq, float* cond, float* pred_next,
                         int replica_budget, int32_t* replicas, int32_t* check, void* stream) {
  using namespace moe;
  if (!dims_ok(L, E, window)) return fail(E > kMaxExperts ? MOE_ERR_UNSUPPORTED : MOE_ERR_INVALID_ARG,
                                          "moe_stats: bad L=%d E=%d window=%d", L, E, window);
  if (!state) return fail(MOE_ERR_INVALID_ARG, "moe_stats: null state");
  if (state_bytes < moe_stats_state_bytes(L, E, window))
    return fail(MOE_ERR_WORKSPACE, "moe_stats: state too small (%zu bytes)", state_bytes);
  if (layer < 0 || layer >= L) return fail(MOE_ERR_INVALID_ARG, "moe_stats: layer=%d outside [0, %d)", layer, L);
  if (iter < 0) return fail(MOE_ERR_INVALID_ARG, "moe_stats: iter < 0");
  if (topk_idx) {
    if (k < 1 || k > E || k > kMaxTopK) return fail(MOE_ERR_INVALID_ARG, "moe_stats: k=%d outside [1, min(E, 8)]", k);
    if (T < 0 || static_cast<int64_t>(window) * T * k * k >= (int64_t(1) << 31))
      return fail(MOE_ERR_INVALID_ARG, "moe_stats: window*T*k*k must stay below 2^31");
    if (layer > 0 && !prev_topk_idx)
      return fail(MOE_ERR_INVALID_ARG, "moe_stats: layer > 0 needs prev_topk_idx");
    if (replicas && (replica_budget < 0 || replica_budget > 4096))
      return fail(MOE_ERR_INVALID_ARG, "moe_stats: replica_budget=%d outside [0, 4096]", replica_budget);
  }
  Args a{};
  a.state = static_cast<int32_t*>(state);
  a.lay = layout(L, E, window);
  a.L = L; a.E = E; a.window = window; a.layer = layer;
  a.slot = static_cast<int>(iter % window);
  a.k = topk_idx ? k : 0;
  a.budget = replica_budget;
  a.T = topk_idx ? T : 0;
  a.idx = topk_idx;
  a.prev = (topk_idx && layer > 0) ? prev_topk_idx : nullptr;
  a.counts = topk_idx ? counts : nullptr;
  a.p_seq = p_seq;
  a.cond = layer + 1 < L ? cond : nullptr;
  a.pred = layer + 1 < L ? pred_next : nullptr;
  a.replicas = topk_idx ? replicas : nullptr;
  a.check = topk_idx ? check : nullptr;
  // E*E beyond the 16-bit LDS counters: 8-bit counters in blocks of fewer tokens
  const bool k8 = topk_idx && layer > 0 && E * E > 2 * kLdsCooc && E * E <= 4 * kLdsCooc;
  const int tpb = k8 ? kTokPerBlock8 : kTokPerBlock;
  const unsigned blocks = topk_idx ? static_cast<unsigned>(std::max<int64_t>(1, ceil_div(T, tpb))) : 1u;
  if (k8) stats_kernel<true><<<blocks, kThreads, 0, as_stream(stream)>>>(a);
  else stats_kernel<false><<<blocks, kThreads, 0, as_stream(stream)>>>(a);
  if (E > kSplitE) {
    const int EE = E * E;
    const int n_ring = (topk_idx && layer > 0) ? static_cast<int>(ceil_div(EE, 8 * kThreads)) : 0;
    const int n_rows = (layer + 1 < L && (a.cond || a.pred)) ? static_cast<int>(ceil_div(E, kThreads / 64)) : 0;
    if (n_ring + n_rows > 0) pair_kernel<<<n_ring + n_rows, kThreads, 0, as_stream(stream)>>>(a, n_ring, n_rows);
  }
  return hip_status(hipGetLastError(), "moe_stats launch");
}

extern "C" int moe_stats_load_state(const void* state, size_t state_bytes, int L, int E, int window, int layer,
                                    int64_t iter, double decay, float* p_decay, int32_t* anomalous,
                                    int32_t* summary, void* stream) {
  using namespace moe;
  if (!dims_ok(L, E, window)) return fail(E > kMaxExperts ? MOE_ERR_UNSUPPORTED : MOE_ERR_INVALID_ARG,
                                          "moe_stats_load_state: bad L=%d E=%d window=%d", L, E, window);
  if (!state) return fail(MOE_ERR_INVALID_ARG, "moe_stats_load_state: null state");
  if (state_bytes < moe_stats_state_bytes(L, E, window))
    return fail(MOE_ERR_WORKSPACE, "moe_stats_load_state: state too small (%zu bytes)", state_bytes);
  if (layer < 0 || layer >= L)
    return fail(MOE_ERR_INVALID_ARG, "moe_stats_load_state: layer=%d outside [0, %d)", layer, L);
  if (iter < 0) return fail(MOE_ERR_INVALID_ARG, "moe_stats_load_state: iter < 0");
  if (!(decay >= 0.0 && decay <= 1.0)) return fail(MOE_ERR_INVALID_ARG, "moe_stats_load_state: decay outside [0, 1]");
  const Layout lay = layout(L, E, window);
  const int m = static_cast<int>(std::min<int64_t>(window, iter + 1));
  load_state_kernel<<<1, kThreads, 0, as_stream(stream)>>>(static_cast<const int32_t*>(state) + lay.cnt_ring, L, E,
                                                            window, layer, static_cast<int>(iter % window), m, decay,
                                                            p_decay, anomalous, summary);
  return hip_status(hipGetLastError(), "moe_stats_load_state launch");
}
