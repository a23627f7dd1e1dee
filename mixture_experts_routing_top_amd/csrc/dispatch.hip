// moe_dispatch: stable expert/replica-contiguous permutation of the tokens.
//
// Source: the token dispatch that precedes the expert computation (EPS-MoE
// review, section 3: tokens go to their experts before the GEMMs, results
// come back for the LocalReduce; PopFetcher wiki, motivation: the dispatch
// All-to-All), done here as a local permute; replica slots follow "Fast MoE
// Inference via Predictive Prefetching and Expert Replication", method
// (physical replicas of one expert serve disjoint subsets of its tokens).
//
// Three launches, no host sync:
//   1. count:   per block of 256 tokens, per-expert counts (LDS atomics) into
//               a [blocks, E] table in the workspace.
//   2. rank:    every block sums the table (all threads, LDS atomics) to get
//               the expert totals, the exclusive expert offsets and its own
//               per-expert prefix;
//               inside the block, each wave ranks its tokens per expert with
//               ballots (order = token order, so the permutation is stable and
//               independent of scheduling).  Block 0 also writes expert_off
//               and the slot table.
//   3. permute: x_perm[inv_pos[t,i]] = x[t], four 16-byte chunks per thread;
//               every source row is read once and written k times, with
//               nontemporal stores (measured ~25% faster than cached stores
//               on this write-heavy copy).
#include "common.h"

namespace {

constexpr int kTok = 256;  // tokens per count/rank block

__global__ __launch_bounds__(kTok) void count_kernel(const int32_t* __restrict__ idx, int64_t T, int k, int E,
                                                     int32_t* __restrict__ blk_cnt) {
  __shared__ int32_t hist[moe::kMaxExperts];
  for (int e = threadIdx.x; e < E; e += kTok) hist[e] = 0;
  __syncthreads();
  const int64_t t = static_cast<int64_t>(blockIdx.x) * kTok + threadIdx.x;
  if (t < T)
    for (int i = 0; i < k; ++i) {
      const int e = idx[t * k + i];
      if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
    }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kTok) blk_cnt[static_cast<int64_t>(blockIdx.x) * E + e] = hist[e];
}

__global__ __launch_bounds__(kTok) void rank_kernel(const int32_t* __restrict__ idx, int64_t T, int k, int E,
                                                    int nblk, const int32_t* __restrict__ blk_cnt,
                                                    const int32_t* __restrict__ replicas, int max_slots,
                                                    int32_t* __restrict__ perm_src, int32_t* __restrict__ inv_pos,
                                                    int32_t* __restrict__ expert_off, int32_t* __restrict__ slot_off,
                                                    int32_t* __restrict__ slot_expert, int32_t* __restrict__ n_slots) {
  __shared__ int32_t tot[moe::kMaxExperts];
  __shared__ int32_t base[moe::kMaxExperts];  // expert offset + this block's prefix
  __shared__ int32_t off[moe::kMaxExperts + 1];
  __shared__ int32_t wave_cnt[kTok / 64][moe::kMaxExperts];
  __shared__ int64_t rep_pre[moe::kMaxExperts + 1];

  const int tid = threadIdx.x;
  const int b = blockIdx.x;
  for (int e = tid; e < E; e += kTok) {
    tot[e] = 0;
    base[e] = 0;
  }
  __syncthreads();
  // every thread reads its share of the [nblk, E] count table (loads in flight
  // together) and adds it into the expert totals and this block's prefix:
  // exact integer sums, so the order of the LDS atomics does not matter
  const int64_t cells = static_cast<int64_t>(nblk) * E;
#pragma unroll 4
  for (int64_t q = tid; q < cells; q += kTok) {
    const int32_t c = blk_cnt[q];
    if (c == 0) continue;
    const int j = static_cast<int>(q / E), e = static_cast<int>(q - static_cast<int64_t>(j) * E);
    atomicAdd(&tot[e], c);
    if (j < b) atomicAdd(&base[e], c);
  }
  __syncthreads();
  if (tid == 0) {  // E <= 256: a short serial scan
    int32_t run = 0;
    for (int e = 0; e < E; ++e) { off[e] = run; run += tot[e]; }
    off[E] = run;
    int64_t rp = 0;
    for (int e = 0; e < E; ++e) { rep_pre[e] = rp; rp += replicas ? max(replicas[e], 0) : 0; }
    rep_pre[E] = rp;
  }
  __syncthreads();
  for (int e = tid; e < E; e += kTok) base[e] += off[e];

  if (b == 0) {
    const int64_t budget = max_slots - E;
    const int32_t M = off[E];
    for (int e = tid; e <= E; e += kTok) expert_off[e] = off[e];
    for (int e = tid; e < E; e += kTok) {
      const int64_t want = replicas ? max(replicas[e], 0) : 0;
      const int64_t r = max<int64_t>(0, min<int64_t>(want, budget - rep_pre[e]));
      const int64_t s0 = e + min<int64_t>(rep_pre[e], budget);
      const int64_t n = tot[e];
      for (int64_t rho = 0; rho <= r; ++rho) {
        slot_expert[s0 + rho] = e;
        slot_off[s0 + rho] = off[e] + static_cast<int32_t>((rho * n) / (r + 1));
      }
    }
    const int64_t used = E + min<int64_t>(rep_pre[E], budget);
    for (int64_t s = used + tid; s <= max_slots; s += kTok) {
      slot_off[s] = M;
      if (s < max_slots) slot_expert[s] = 0;
    }
    if (tid == 0) n_slots[0] = static_cast<int32_t>(used);
  }

  // Rank inside the block: wave w ranks its 64 tokens per expert with ballots.
  const int64_t t = static_cast<int64_t>(b) * kTok + tid;
  const bool active = t < T;
  const int lane = tid & 63, w = tid >> 6;
  int cur[moe::kMaxTopK];
  int rk[moe::kMaxTopK];
#pragma unroll
  for (int i = 0; i < moe::kMaxTopK; ++i) {
    cur[i] = -1;
    rk[i] = 0;
    if (active && i < k) {
      const int e = idx[t * k + i];
      cur[i] = (e >= 0 && e < E) ? e : -1;
    }
  }
  const uint64_t lt = (uint64_t(1) << lane) - 1;
  for (int e = 0; e < E; ++e) {
    bool has = false;
#pragma unroll
    for (int i = 0; i < moe::kMaxTopK; ++i) has |= (cur[i] == e);
    const uint64_t m = __ballot(has);
    if (m == 0) {
      if (lane == 0) wave_cnt[w][e] = 0;
      continue;
    }
    const int r = __popcll(m & lt);
#pragma unroll
    for (int i = 0; i < moe::kMaxTopK; ++i)
      if (cur[i] == e) rk[i] = r;
    if (lane == 0) wave_cnt[w][e] = __popcll(m);
  }
  __syncthreads();
  if (!active) return;
#pragma unroll
  for (int i = 0; i < moe::kMaxTopK; ++i) {
    if (i >= k) break;
    const int e = cur[i];
    if (e < 0) {
      inv_pos[t * k + i] = -1;
      continue;
    }
    int32_t row = base[e] + rk[i];
    for (int v = 0; v < w; ++v) row += wave_cnt[v][e];
    perm_src[row] = static_cast<int32_t>(t);
    inv_pos[t * k + i] = row;
  }
}

// Four 16-byte chunks of one source row per thread (strided so a wave's
// accesses stay contiguous); each chunk is read once and written to the k
// destination rows.
constexpr int kChunksPerThread = 4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void permute_kernel(const uint4* __restrict__ x, int64_t T, int chunks, int k,
                                                      int64_t M, const int32_t* __restrict__ inv_pos,
                                                      uint4* __restrict__ x_perm) {
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
    const int32_t r = inv_pos[t * k + i];
    if (r < 0 || r >= M) continue;
    uint4* dst = x_perm + static_cast<int64_t>(r) * chunks;
#pragma unroll
    for (int u = 0; u < kChunksPerThread; ++u) {
      const int c = c0 + u * groups;
      if (c < chunks)
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&v[u]), reinterpret_cast<u32x4*>(dst + c));
    }
  }
}

}  // namespace

extern "C" size_t moe_dispatch_workspace_bytes(int64_t T, int k, int E) {
  (void)k;
  if (T < 0 || E < 1) return 0;
  return moe::align_up(static_cast<size_t>(std::max<int64_t>(1, moe::ceil_div(T, kTok))) * E * sizeof(int32_t), 256);
}

extern "C" int moe_dispatch(const void* x, moe_dtype dt, int64_t T, int H, const int32_t* topk_idx, int k, int E,
                            const int32_t* replicas, int max_slots,
                            void* x_perm, int32_t* perm_src, int32_t* inv_pos, int32_t* expert_off,
                            int32_t* slot_off, int32_t* slot_expert, int32_t* n_slots,
                            void* workspace, size_t workspace_bytes, void* stream) {
  using namespace moe;
  if (E < 1 || E > kMaxExperts) return fail(E < 1 ? MOE_ERR_INVALID_ARG : MOE_ERR_UNSUPPORTED,
                                            "moe_dispatch: E=%d outside [1, %d]", E, kMaxExperts);
  if (k < 1 || k > E || k > kMaxTopK) return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: k=%d outside [1, min(E, 8)]", k);
  if (T < 0 || T * k >= (int64_t(1) << 31)) return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: T*k must stay below 2^31");
  if (dt != MOE_F32 && dt != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: unknown dtype %d", (int)dt);
  if (H < 1 || (static_cast<int64_t>(H) * elem_bytes(dt)) % 16 != 0)
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: H*sizeof(dtype) must be a positive multiple of 16 (H=%d)", H);
  if (max_slots < E || max_slots > E + 65536) return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: max_slots=%d outside [E, E+65536]", max_slots);
  if (!expert_off || !slot_off || !slot_expert || !n_slots || !workspace)
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: null pointer");
  if (T > 0 && (!x || !topk_idx || !x_perm || !perm_src || !inv_pos))
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: null pointer");
  if (T > 0 && (!aligned16(x) || !aligned16(x_perm)))
    return fail(MOE_ERR_INVALID_ARG, "moe_dispatch: x and x_perm must be 16-byte aligned");
  if (workspace_bytes < moe_dispatch_workspace_bytes(T, k, E))
    return fail(MOE_ERR_WORKSPACE, "moe_dispatch: workspace has %zu bytes, needs %zu", workspace_bytes,
                moe_dispatch_workspace_bytes(T, k, E));
  const hipStream_t s = as_stream(stream);
  int32_t* blk_cnt = static_cast<int32_t*>(workspace);
  const int nblk = static_cast<int>(ceil_div(T, kTok));
  if (nblk > 0) count_kernel<<<nblk, kTok, 0, s>>>(topk_idx, T, k, E, blk_cnt);
  rank_kernel<<<std::max(nblk, 1), kTok, 0, s>>>(topk_idx, T, k, E, nblk, blk_cnt, replicas, max_slots, perm_src,
                                                 inv_pos, expert_off, slot_off, slot_expert, n_slots);
  if (T > 0) {
    const int chunks = static_cast<int>(static_cast<int64_t>(H) * elem_bytes(dt) / 16);
    const int64_t threads = T * ceil_div(chunks, kChunksPerThread);
    permute_kernel<<<static_cast<unsigned>(ceil_div(threads, 256)), 256, 0, s>>>(
        static_cast<const uint4*>(x), T, chunks, k, T * k, inv_pos, static_cast<uint4*>(x_perm));
  }
  return hip_status(hipGetLastError(), "moe_dispatch launch");
}
