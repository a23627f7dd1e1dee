// moe_dispatch: stable expert/replica-contiguous permutation of the tokens.
//
// Source: the token dispatch that precedes the expert computation (EPS-MoE
// review, section 3: tokens go to their experts before the GEMMs, results
// come back for the LocalReduce; PopFetcher wiki, motivation: the dispatch
// All-to-All), done here as a local permute; replica slots follow "Fast MoE
// Inference via Predictive Prefetching and Expert Replication", method
// (physical replicas of one expert serve disjoint subsets of its tokens).
//
// The (token, slot) pairs are numbered f = t*k + i; inside an expert the rows
// follow ascending f (ascending token index; a token naming one expert twice
// gets two rows in slot order).  Small dispatches (up to 1024 pairs over up to
// 64 experts) run in one launch (dispatch_small_kernel, plus the copy when
// asked for); the others in three launches, no host sync:
//   1. rank:    per block of kPairs pairs, its per-expert counts (into a
//               [blocks, E] table) and each pair's rank among the block's
//               pairs of the same expert: wave ballots over the distinct
//               experts of a wave, LDS counts across waves and rounds.
//   2. scan:    one block: the expert totals, expert_off, and per block and
//               expert the first row of the block's pairs (the column prefix
//               of the count table, O(blocks x E)); the replica plan from the
//               totals when asked for (replica_budget); the slot table; with a
//               check word, the totals against `counts` and the replicas
//               against the slot budget.
//   3. permute: row = base[f / kPairs][e] + rank[f]; the threads of token t
//               write inv_pos and perm_src and copy x[t] into each of its
//               rows: four 16-byte chunks per thread, read once, written k
//               times with nontemporal stores (measured ~25% faster than cached
//               stores on this write-heavy copy).  Without x_perm only the
//               indices are written (the expert FFN can gather its rows from
//               x through perm_src instead).
#include <mutex>

#include "common.h"
#include "replica_plan.h"

namespace {

constexpr int kThreads = 256;
// the one scan block: NT / E threads per expert column; NT = 1024 for count
// tables of more than kWideScan entries (the DeepSeek-V2 shape), 256 below (a
// 1024-thread block costs a few microseconds more where there is little to sum)
constexpr int kWideScan = 2048;
constexpr int kPairs = 512;  // pairs per rank block (two rounds of 256)
static_assert(kPairs % kThreads == 0, "whole rounds");

struct Ws {
  size_t cnt, base, rank, bytes;
};

Ws ws_layout(int64_t T, int k, int E) {
  Ws w{};
  const int64_t P = T * k;
  const int64_t nblk = std::max<int64_t>(1, moe::ceil_div(P, kPairs));
  size_t at = 0;
  auto take = [&](size_t n) { size_t p = at; at = moe::align_up(at + n, 256); return p; };
  w.cnt = take(static_cast<size_t>(nblk) * E * sizeof(int32_t));
  w.base = take(static_cast<size_t>(nblk) * E * sizeof(int32_t));
  w.rank = take(static_cast<size_t>(std::max<int64_t>(P, 1)) * sizeof(int32_t));
  w.bytes = at;
  return w;
}

__global__ __launch_bounds__(kThreads) void rank_kernel(const int32_t* __restrict__ idx, int64_t P, int k, int E,
                                                        int32_t* __restrict__ blk_cnt, int32_t* __restrict__ rank,
                                                        int32_t* __restrict__ check) {
  __shared__ int32_t run[moe::kMaxExperts];                  // this block's pairs so far, per expert
  __shared__ int32_t wave_cnt[kThreads / 64][moe::kMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int e = tid; e < E; e += kThreads) run[e] = 0;
  const int64_t f0 = static_cast<int64_t>(blockIdx.x) * kPairs;
  const uint64_t lt = (uint64_t(1) << lane) - 1;
  bool bad_index = false, bad_dup = false;
  for (int r = 0; r < kPairs / kThreads; ++r) {
    for (int q = tid; q < (kThreads / 64) * moe::kMaxExperts; q += kThreads) (&wave_cnt[0][0])[q] = 0;
    const int64_t f = f0 + r * kThreads + tid;
    int e = -1;
    if (f < P) {
      e = idx[f];
      if (e < 0 || e >= E) {
        bad_index = true;
        e = -1;
      } else if (check) {
        const int64_t t = f / k;
        for (int64_t j = t * k; j < f; ++j) bad_dup |= idx[j] == e;
      }
    }
    __syncthreads();
    // rank inside the wave: one ballot per distinct expert of the wave (the
    // leader's expert read with v_readlane: the leader is wave-uniform)
    int local = 0;
    uint64_t todo = __ballot(e >= 0);
    while (todo) {
      const int leader = __ffsll(static_cast<unsigned long long>(todo)) - 1;
      const int v = __builtin_amdgcn_readlane(e, leader);
      const uint64_t m = __ballot(e == v);
      if (e == v) local = __popcll(m & lt);
      if (lane == leader) wave_cnt[w][v] = __popcll(m);
      todo &= ~m;
    }
    __syncthreads();
    if (e >= 0) {
      int rk = run[e] + local;
      for (int v = 0; v < w; ++v) rk += wave_cnt[v][e];
      rank[f] = rk;
    }
    __syncthreads();
    for (int x = tid; x < E; x += kThreads)
      run[x] += wave_cnt[0][x] + wave_cnt[1][x] + wave_cnt[2][x] + wave_cnt[3][x];
    __syncthreads();
  }
  for (int e = tid; e < E; e += kThreads) blk_cnt[static_cast<int64_t>(blockIdx.x) * E + e] = run[e];
  if (check) {
    raise_check(check, bad_index, MOE_CHECK_INDEX);
    raise_check(check, bad_dup, MOE_CHECK_DUPLICATE);
  }
}

// Inclusive prefix sum over the block's first n <= 256 values of v (in place,
// LDS), every thread of the block taking part.
__device__ void block_scan_inclusive(int64_t* v, int n) {
  const int tid = threadIdx.x;
  for (int d = 1; d < n; d <<= 1) {
    const int64_t add = (tid < n && tid >= d) ? v[tid - d] : 0;
    __syncthreads();
    if (tid < n) v[tid] += add;
    __syncthreads();
  }
}

// The expert totals `tot` (LDS) become the layer's offsets and slot table:
// the replica plan from the totals when asked for (plan_budget), expert_off,
// the slot table, and with a check word the totals against `counts` and the
// replicas against the slot budget.  Leaves off[e] = inclusive prefix of the
// totals (LDS) for the caller.  Every thread of the block takes part.
__device__ void offsets_and_slots(const int32_t* tot, int64_t* off, int64_t* rep, int32_t* want_s, int E, int64_t P,
                                  const int32_t* __restrict__ counts, const int32_t* __restrict__ replicas,
                                  int plan_budget, int max_slots, int32_t* __restrict__ expert_off,
                                  int32_t* __restrict__ slot_off, int32_t* __restrict__ slot_expert,
                                  int32_t* __restrict__ n_slots, int32_t* __restrict__ check) {
  const int tid = threadIdx.x, nt = blockDim.x;
  if (tid < E) {
    off[tid] = tot[tid];
    want_s[tid] = replicas ? replicas[tid] : 0;
  }
  __syncthreads();
  // this routing's replica plan (wave 0: 64 lanes x 4 experts; total = T*k)
  if (plan_budget > 0 && tid < 64) {
    int64_t n[4];
    int r[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) n[j] = tid + 64 * j < E ? tot[tid + 64 * j] : 0;
    moe::plan_replicas_wave(n, E, P, plan_budget, tid, r);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (tid + 64 * j < E) want_s[tid + 64 * j] = r[j];
  }
  __syncthreads();
  if (tid < E) rep[tid] = max(want_s[tid], 0);
  __syncthreads();
  // exclusive prefixes: expert offsets and replica counts
  block_scan_inclusive(off, E);
  block_scan_inclusive(rep, E);
  const int32_t M = E > 0 ? static_cast<int32_t>(off[E - 1]) : 0;
  // expert offsets and the slot table
  const int64_t budget = max_slots - E;
  bool bad_counts = false, bad_reps = false;
  for (int x = tid; x < E; x += nt) {
    const int64_t excl = off[x] - tot[x];
    expert_off[x] = static_cast<int32_t>(excl);
    const int64_t want = max(want_s[x], 0);
    const int64_t rp = rep[x] - want;  // copies of experts before x
    const int64_t r = max<int64_t>(0, min<int64_t>(want, budget - rp));
    const int64_t s0 = x + min<int64_t>(rp, budget);
    const int64_t n = tot[x];
    for (int64_t rho = 0; rho <= r; ++rho) {
      slot_expert[s0 + rho] = x;
      slot_off[s0 + rho] = static_cast<int32_t>(excl + (rho * n) / (r + 1));
    }
    bad_counts |= counts && counts[x] != tot[x];
    bad_reps |= want_s[x] < 0 || r < want;
  }
  if (tid == 0) expert_off[E] = M;
  const int64_t all = E > 0 ? rep[E - 1] : 0;
  const int64_t used = E + min<int64_t>(all, budget);
  for (int64_t q = used + tid; q <= max_slots; q += nt) {
    slot_off[q] = M;
    if (q < max_slots) slot_expert[q] = 0;
  }
  if (tid == 0) n_slots[0] = static_cast<int32_t>(used);
  if (check) {
    raise_check(check, bad_counts, MOE_CHECK_COUNTS);
    raise_check(check, bad_reps, MOE_CHECK_REPLICAS);
  }
}

template <int kScanThreads>
__global__ __launch_bounds__(kScanThreads) void scan_kernel(const int32_t* __restrict__ blk_cnt, int nblk, int E,
                                                        int64_t P, const int32_t* __restrict__ counts,
                                                        const int32_t* __restrict__ replicas, int plan_budget,
                                                        int max_slots,
                                                        int32_t* __restrict__ blk_base, int32_t* __restrict__ expert_off,
                                                        int32_t* __restrict__ slot_off,
                                                        int32_t* __restrict__ slot_expert, int32_t* __restrict__ n_slots,
                                                        int32_t* __restrict__ check) {
  __shared__ int32_t part[kScanThreads];   // [group][expert] partial column sums
  __shared__ int64_t off[moe::kMaxExperts];
  __shared__ int64_t rep[moe::kMaxExperts];
  __shared__ int32_t tot[moe::kMaxExperts];
  __shared__ int32_t want_s[moe::kMaxExperts];   // replicas asked for, per expert
  const int tid = threadIdx.x;
  // thread (g, e) = g*E + e sums column e over group g's run of blocks, eight
  // loads in flight
  constexpr int U = 8;
  const int G = max(1, min(kScanThreads / E, nblk));  // no more groups than blocks
  const int g = tid / E, e = tid - g * E;
  const int per = (nblk + G - 1) / G;
  const int b0 = min(g * per, nblk), b1 = min(b0 + per, nblk);
  int32_t s = 0;
  if (g < G) {
    for (int b = b0; b < b1; b += U) {
      int32_t c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) c[u] = b + u < b1 ? blk_cnt[static_cast<int64_t>(b + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u) s += c[u];
    }
    part[tid] = s;
  }
  __syncthreads();
  if (tid < E) {
    int32_t t = 0;
    for (int q = 0; q < G; ++q) t += part[q * E + tid];
    tot[tid] = t;
  }
  __syncthreads();
  offsets_and_slots(tot, off, rep, want_s, E, P, counts, replicas, plan_budget, max_slots, expert_off, slot_off,
                    slot_expert, n_slots, check);
  // group prefix of each column, then this group's blocks
  if (g < G) {
    int32_t run = static_cast<int32_t>(off[e] - tot[e]);
    for (int q = 0; q < g; ++q) run += part[q * E + e];
    for (int b = b0; b < b1; b += U) {
      int32_t c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) c[u] = b + u < b1 ? blk_cnt[static_cast<int64_t>(b + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (b + u < b1) blk_base[static_cast<int64_t>(b + u) * E + e] = run;
        run += c[u];
      }
    }
  }
}

// Small dispatches (at most kSmallPairs pairs, at most kSmallExperts experts)
// in one launch of one block, where the three launches below would cost more
// in launch latency than they do work.  Wave w takes a contiguous run of C
// pairs (C a multiple of 64, 16 C >= P), so the pairs keep their ascending
// order as (wave, round of 64, lane).  Each wave counts its run's experts with
// one ballot per distinct expert of a round, lane v keeping expert v's count in
// a register (E <= 64); the block turns the totals into offsets and slots
// (offsets_and_slots); each expert's column of the [wave, expert] table of
// counts becomes the first row of each wave's pairs of that expert; and each
// wave ranks its run again with the same ballots, lane v holding and advancing
// the wave's next row of expert v.  The rows are those of the three-launch
// path, with no workspace.
constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / 64;
// rounds of 64 pairs per wave: one.  A round costs each wave one ballot per
// distinct expert of its 64 pairs, twice, and the block's 16 waves share one CU
// where the three-launch path spreads its rank blocks over many: measured per
// call, T*k = 512 and 1024 (E = 8) took 8.5 and 9.7 us against 12.3 and 13.1 us
// in three launches, T*k = 4096 took 14.8 / 25.5 / 23.9 us (E = 8 / 32 / 64)
// against 14.2 / 19.6 / 13.1 us.
constexpr int kSmallRounds = 1;
constexpr int64_t kSmallPairs = int64_t(kSmallThreads) * kSmallRounds;
constexpr int kSmallExperts = 64;  // a round's ballots are at most min(E, 64)

__global__ __launch_bounds__(kSmallThreads) void dispatch_small_kernel(
    const int32_t* __restrict__ idx, int64_t P, int k, int E, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ replicas, int plan_budget, int max_slots, int32_t* __restrict__ expert_off,
    int32_t* __restrict__ slot_off, int32_t* __restrict__ slot_expert, int32_t* __restrict__ n_slots,
    int32_t* __restrict__ perm_src, int32_t* __restrict__ inv_pos, int32_t* __restrict__ check) {
  __shared__ int64_t off[moe::kMaxExperts];
  __shared__ int64_t rep[moe::kMaxExperts];
  __shared__ int32_t tot[moe::kMaxExperts];
  __shared__ int32_t want_s[moe::kMaxExperts];
  __shared__ int32_t wtab[kSmallWaves][kSmallExperts];  // per wave: its counts, then its next rows
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int q = tid; q < kSmallWaves * kSmallExperts; q += kSmallThreads) (&wtab[0][0])[q] = 0;
  const int C = static_cast<int>((P + kSmallThreads - 1) / kSmallThreads) * 64;  // pairs per wave
  const int rounds = C / 64;                                                      // <= kSmallRounds
  int ev[kSmallRounds];
  bool bad_index = false, bad_dup = false;
#pragma unroll
  for (int r = 0; r < kSmallRounds; ++r) {
    const int64_t f = static_cast<int64_t>(w) * C + r * 64 + lane;
    int e = -1;
    if (r < rounds && f < P) {
      e = idx[f];
      if (e < 0 || e >= E) {
        bad_index = true;
        e = -1;
      } else if (check) {
        const int64_t t = f / k;
        for (int64_t j = t * k; j < f; ++j) bad_dup |= idx[j] == e;
      }
    }
    ev[r] = e;
  }
  __syncthreads();
  const uint64_t lt = (uint64_t(1) << lane) - 1;
  // pass 1: this wave's counts, lane v counting expert v (E <= 64) in a register
  int32_t cnt = 0;
#pragma unroll
  for (int r = 0; r < kSmallRounds; ++r) {
    const int e = ev[r];
    uint64_t todo = __ballot(e >= 0);
    while (todo) {
      const int leader = __ffsll(static_cast<unsigned long long>(todo)) - 1;
      const int v = __builtin_amdgcn_readlane(e, leader);
      const uint64_t m = __ballot(e == v);
      if (lane == v) cnt += __popcll(m);
      todo &= ~m;
    }
  }
  if (lane < E) wtab[w][lane] = cnt;
  __syncthreads();
  for (int x = tid; x < E; x += kSmallThreads) {
    int32_t t = 0;
#pragma unroll
    for (int v = 0; v < kSmallWaves; ++v) t += wtab[v][x];
    tot[x] = t;
  }
  __syncthreads();
  offsets_and_slots(tot, off, rep, want_s, E, P, counts, replicas, plan_budget, max_slots, expert_off, slot_off,
                    slot_expert, n_slots, check);
  // each expert's column: the first row of every wave's pairs of that expert
  for (int x = tid; x < E; x += kSmallThreads) {
    int32_t row = static_cast<int32_t>(off[x] - tot[x]);
#pragma unroll
    for (int v = 0; v < kSmallWaves; ++v) {
      const int32_t c = wtab[v][x];
      wtab[v][x] = row;
      row += c;
    }
  }
  __syncthreads();
  // pass 2: this wave's rows, in pair order; lane v holds the wave's next row
  // of expert v
  int32_t next = lane < E ? wtab[w][lane] : 0;
#pragma unroll
  for (int r = 0; r < kSmallRounds; ++r) {
    const int64_t f = static_cast<int64_t>(w) * C + r * 64 + lane;
    const int e = ev[r];
    int32_t row = -1;
    uint64_t todo = __ballot(e >= 0);
    while (todo) {
      const int leader = __ffsll(static_cast<unsigned long long>(todo)) - 1;
      const int v = __builtin_amdgcn_readlane(e, leader);
      const uint64_t m = __ballot(e == v);
      const int32_t base = __builtin_amdgcn_readlane(next, v);
      if (e == v) row = base + __popcll(m & lt);
      if (lane == v) next += __popcll(m);
      todo &= ~m;
    }
    if (r < rounds && f < P) {
      inv_pos[f] = row;
      if (row >= 0) perm_src[row] = static_cast<int32_t>(f / k);
    }
  }
  if (check) {
    raise_check(check, bad_index, MOE_CHECK_INDEX);
    raise_check(check, bad_dup, MOE_CHECK_DUPLICATE);
  }
}

// Four 16-byte chunks of one source row per thread (strided so a wave's
// accesses stay contiguous); each chunk is read once and written to the k
// destination rows.  The thread holding chunk group 0 of a token also writes
// the token's inv_pos entries and perm_src of its rows.
constexpr int kChunksPerThread = 4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// kFromInv: the rows come from inv_pos, which dispatch_small_kernel has written
// (as it has perm_src); blk_base and rank are not read.
template <bool kFromInv>
__global__ __launch_bounds__(256) void permute_kernel(const uint4* __restrict__ x, int64_t T, int chunks, int k, int E,
                                                      const int32_t* __restrict__ idx,
                                                      const int32_t* __restrict__ blk_base,
                                                      const int32_t* __restrict__ rank, int32_t* __restrict__ perm_src,
                                                      int32_t* __restrict__ inv_pos, uint4* __restrict__ x_perm) {
  const int groups = (chunks + kChunksPerThread - 1) / kChunksPerThread;
  const int64_t g = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (g >= T * groups) return;
  const int64_t t = g / groups;
  const int c0 = static_cast<int>(g - t * groups);
  uint4 v[kChunksPerThread];
#pragma unroll
  for (int u = 0; u < kChunksPerThread; ++u) {
    const int c = c0 + u * groups;
    if (c < chunks) v[u] = x[t * chunks + c];
  }
  for (int i = 0; i < k; ++i) {
    const int64_t f = t * k + i;
    int32_t r;
    if constexpr (kFromInv) {
      r = inv_pos[f];
    } else {
      const int e = idx[f];
      r = (e >= 0 && e < E) ? blk_base[(f / kPairs) * E + e] + rank[f] : -1;
      if (c0 == 0) {
        inv_pos[f] = r;
        if (r >= 0) perm_src[r] = static_cast<int32_t>(t);
      }
    }
    if (r < 0) continue;
    uint4* dst = x_perm + static_cast<int64_t>(r) * chunks;
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
      const int c = c0 + u * groups;
      if (c < chunks)
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&v[u]), reinterpret_cast<u32x4*>(dst + c));
    }
  }
}

// Without a row copy (x_perm NULL): one thread per (token, slot) pair writes
// its inv_pos and its row's perm_src.
__global__ __launch_bounds__(256) void index_kernel(int64_t P, int k, int E, const int32_t* __restrict__ idx,
                                                    const int32_t* __restrict__ blk_base,
                                                    const int32_t* __restrict__ rank, int32_t* __restrict__ perm_src,
                                                    int32_t* __restrict__ inv_pos) {
  const int64_t f = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (f >= P) return;
  const int e = idx[f];
  const int32_t r = (e >= 0 && e < E) ? blk_base[(f / kPairs) * E + e] + rank[f] : -1;
  inv_pos[f] = r;
  if (r >= 0) perm_src[r] = static_cast<int32_t>(f / k);
}

// Device scratch of moe_dispatch_noalloc: the workspace of one call, in a
// file-scope array each GPU holds for the life of the process (8 MiB: up to
// 2^20 (token, slot) pairs at E = 256).  Host code uses it only through the
// address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the current device, looked up once per device.
int scratch_on_current_device(void** out) {
  int dev = -1;
  if (int rc = moe::hip_status(hipGetDevice(&dev), "moe_dispatch_noalloc hipGetDevice")) return rc;
  if (dev < 0 || dev >= kMaxDevices) return moe::fail(MOE_ERR_UNSUPPORTED, "moe_dispatch_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (int rc = moe::hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "moe_dispatch_noalloc scratch"))
      return rc;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" size_t moe_dispatch_workspace_bytes(int64_t T, int k, int E) {
  if (T < 0 || E < 1 || E > moe::kMaxExperts || k < 1 || k > moe::kMaxTopK) return 0;
  return ws_layout(T, k, E).bytes;
}

extern "C" int moe_dispatch(const void* x, moe_dtype dt, int64_t T, int H, const int32_t* topk_idx, int k, int E,
                            const int32_t* counts, const int32_t* replicas, int replica_budget, int max_slots,
                            void* x_perm, int32_t* perm_src, int32_t* inv_pos, int32_t* expert_off,
                            int32_t* slot_off, int32_t* slot_expert, int32_t* n_slots,
                            void* workspace, size_t workspace_bytes, int32_t* check, void* stream) {
  using namespace moe;
  if (E < 1 || E > kMaxExperts) return fail(E < 1 ? MOE_ERR_INVALID_ARG : MOE_ERR_UNSUPPORTED,
                                            "moe_dispatch: E=%d outside [1, %d]", E, kMaxExperts);
  if (k < 1 || k > E || k > kMaxTopK) return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: k=%d outside [1, min(E, 8)]", k);
  if (T < 0 || T * k >= (int64_t(1) << 31)) return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: T*k must stay below 2^31");
  if (dt != MOE_F32 && dt != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: unknown dtype %d", (int)dt);
  if (H < 1 || (static_cast<int64_t>(H) * elem_bytes(dt)) % 16 != 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: H*sizeof(dtype) must be a positive multiple of 16 (H=%d)", H);
  if (max_slots < E || max_slots > E + 65536) return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: max_slots=%d outside [E, E+65536]", max_slots);
  if (replica_budget < 0 || replica_budget > max_slots - E || (replicas && replica_budget != 0))
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: replica_budget=%d must lie in [0, max_slots - E] and be 0 "
                "when replicas is given", replica_budget);
  if (!expert_off || !slot_off || !slot_expert || !n_slots || !workspace)
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: null pointer");
  if (T > 0 && (!topk_idx || !perm_src || !inv_pos || (x_perm && !x)))
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: null pointer");
  if (T > 0 && x_perm && (!aligned16(x) || !aligned16(x_perm)))
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: x and x_perm must be 16-byte aligned");
  const Ws w = ws_layout(T, k, E);
  if (workspace_bytes < w.bytes)
    return fail(MOE_ERR_WORKSPACE, "moe_dispatch: workspace has %zu bytes, needs %zu", workspace_bytes, w.bytes);
  const hipStream_t s = as_stream(stream);
  char* ws = static_cast<char*>(workspace);
  int32_t* blk_cnt = reinterpret_cast<int32_t*>(ws + w.cnt);
  int32_t* blk_base = reinterpret_cast<int32_t*>(ws + w.base);
  int32_t* rank = reinterpret_cast<int32_t*>(ws + w.rank);
  const int64_t P = T * k;
  const int chunks = static_cast<int>(static_cast<int64_t>(H) * elem_bytes(dt) / 16);
  const int64_t copy_threads = T * ceil_div(chunks, kChunksPerThread);
  if (P <= kSmallPairs && E <= kSmallExperts) {
    dispatch_small_kernel<<<1, kSmallThreads, 0, s>>>(topk_idx, P, k, E, counts, replicas, replica_budget, max_slots,
                                                      expert_off, slot_off, slot_expert, n_slots, perm_src, inv_pos,
                                                      check);
    if (T > 0 && x_perm)
      permute_kernel<true><<<static_cast<unsigned>(ceil_div(copy_threads, 256)), 256, 0, s>>>(
          static_cast<const uint4*>(x), T, chunks, k, E, topk_idx, nullptr, nullptr, perm_src, inv_pos,
          static_cast<uint4*>(x_perm));
    return hip_status(hipGetLastError(), "moe_dispatch launch");
  }
  const int nblk = static_cast<int>(ceil_div(P, kPairs));
  if (nblk > 0) rank_kernel<<<nblk, kThreads, 0, s>>>(topk_idx, P, k, E, blk_cnt, rank, check);
  if (static_cast<int64_t>(nblk) * E > kWideScan)
    scan_kernel<1024><<<1, 1024, 0, s>>>(blk_cnt, nblk, E, P, counts, replicas, replica_budget, max_slots, blk_base,
                                         expert_off, slot_off, slot_expert, n_slots, check);
  else
    scan_kernel<256><<<1, 256, 0, s>>>(blk_cnt, nblk, E, P, counts, replicas, replica_budget, max_slots, blk_base,
                                       expert_off, slot_off, slot_expert, n_slots, check);
  if (T > 0 && x_perm) {
    permute_kernel<false><<<static_cast<unsigned>(ceil_div(copy_threads, 256)), 256, 0, s>>>(
        static_cast<const uint4*>(x), T, chunks, k, E, topk_idx, blk_base, rank, perm_src, inv_pos,
        static_cast<uint4*>(x_perm));
  } else if (T > 0) {
    index_kernel<<<static_cast<unsigned>(ceil_div(P, 256)), 256, 0, s>>>(P, k, E, topk_idx, blk_base, rank,
                                                                          perm_src, inv_pos);
  }
  return hip_status(hipGetLastError(), "moe_dispatch launch");
}

extern "C" int moe_dispatch_noalloc(const void* x, moe_dtype dt, int64_t T, int H, const int32_t* topk_idx, int k,
                                    int E, const int32_t* counts, const int32_t* replicas, int replica_budget,
                                    int max_slots, void* x_perm,
                                    int32_t* perm_src, int32_t* inv_pos, int32_t* expert_off, int32_t* slot_off,
                                    int32_t* slot_expert, int32_t* n_slots, int32_t* check, void* stream) {
  using namespace moe;
  if (E >= 1 && E <= kMaxExperts && k >= 1 && k <= kMaxTopK && T >= 0 && T * k < (int64_t(1) << 31)) {
    const size_t need = ws_layout(T, k, E).bytes;
    if (need > kScratchBytes)
      return fail(MOE_ERR_WORKSPACE, "moe_dispatch_noalloc: T=%lld, k=%d, E=%d needs %zu bytes of scratch; the "
                  "static scratch holds %zu (use moe_dispatch with a workspace)", (long long)T, k, E, need,
                  kScratchBytes);
  }
  void* ws = nullptr;
  if (int rc = scratch_on_current_device(&ws)) return rc;
  return moe_dispatch(x, dt, T, H, topk_idx, k, E, counts, replicas, replica_budget, max_slots, x_perm, perm_src,
                      inv_pos, expert_off, slot_off, slot_expert, n_slots, ws, kScratchBytes, check, stream);
}
