// moe_expert_ffn: the experts' FFNs over the slot-contiguous rows, as grouped
// GEMMs on the MI355X matrix cores.
//
// Source: EPS-MoE review, section 3 (the gate, up and down GEMMs are the
// compute-bound part of an MoE layer; GroupGemm runs every expert's product in
// one kernel; DenseGemm runs a padded uniform batch and wins at small counts).
// SwiGLU h = silu(x Wg^T) * (x Wu^T), y = h Wd^T; GELU h = gelu(x W1^T),
// y = h W2^T.
//
// A tile-table pass, then two launches of one tiled kernel:
//   tiles:   lists every (slot, 256-row tile); tiles cover each slot's rows
//            exactly, no host sync.
//   phase 1: per tile and per 128 columns of I, the gate and up weight tiles
//            are multiplied side by side so one lane holds g and u of the same
//            element; the activation runs in the epilogue and h is rounded to
//            the dtype once (GELU: one 256-column weight tile).
//   phase 2: y = h Wd^T per tile and 256 columns of H, rounded to the dtype.
//
// gfx950 mapping.  A block is 256 threads (4 waves, one per SIMD) computing a
// 256 x 256 output tile; each wave owns 128 x 128 as 4 x 4 MFMA tiles of
// 32 x 32 (v_mfma_f32_32x32x16_bf16, or v_mfma_f32_32x32x2f32 for fp32), 256
// accumulator registers.  K advances 128 bytes per row per step (64 bf16 / 32
// fp32) through two LDS stages (2 x 144 KB-ish of padded rows, conflict-free
// 16-byte fragment reads); the next step's tiles travel global -> registers
// while the current one is multiplied, one barrier per step.  Operands are
// read with raw buffer loads whose range ends at the slot's (or matrix's)
// last valid row, so rows past the end read as zero and need no clamping.
// Blocks are remapped so each of the 8 XCDs works on a contiguous run of
// tiles, ordered 8 row tiles by N columns, which keeps the A and B tiles that
// neighbouring blocks share inside that XCD's L2.  Each output row depends
// only on its own input row and the fixed K order, so a row's value does not
// depend on the tile, slot or path that computes it.
#include <algorithm>
#include <vector>

#include "common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

enum Epi { kEpiSwiGLU = 0, kEpiGELU = 1, kEpiStore = 2 };

template <bool kBf16>
struct Tr;
template <>
struct Tr<true> {
  using T = uint16_t;
  static constexpr int BK = 64;  // K elements per step (128 bytes per row)
  static constexpr int MK = 16;  // K per MFMA
  static constexpr int KV = 8;   // K elements per lane per MFMA
  using Frag = uint4;
};
template <>
struct Tr<false> {
  using T = float;
  static constexpr int BK = 32;
  static constexpr int MK = 2;
  static constexpr int KV = 1;
  using Frag = float;
};

__device__ __forceinline__ f32x16 mma(const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}
__device__ __forceinline__ f32x16 mma(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

constexpr int kTileN = 256;      // weight rows per tile (gate/up: 128 + 128)
constexpr int kRowBytes = 144;   // LDS row pitch: 128 data bytes + 16 pad
constexpr int kGroupM = 8;       // row tiles per raster group

struct GemmArgs {
  const void* A;   // [M, K]
  const void* B0;  // [E, N, K]
  const void* B1;  // [E, N, K] or null
  void* C;         // [M, N]
  int64_t M;
  int K, N, E;
  const int32_t* slot_off;
  const int32_t* slot_expert;
  const int32_t* tile_slot;
  const int32_t* tile_row0;
  const int32_t* n_tiles;
  int n_col_tiles;
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : static_cast<int>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n, 0x00020000);
}

__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// BM rows x 256 weight rows per block; the 4 waves form a WM x (4/WM) grid.
// BM = 256, WM = 2: each wave owns 128 x 128 (4 x 4 MFMA tiles).
// BM = 64,  WM = 1: each wave owns  64 x 64  (2 x 2 MFMA tiles).
template <bool kBf16, int NMAT, int EPI, int BM, int WM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_kernel(GemmArgs g) {
  using TR = Tr<kBf16>;
  using T = typename TR::T;
  using Frag = typename TR::Frag;
  constexpr int S = sizeof(T);
  constexpr int BK = TR::BK;
  constexpr int KS = BK / TR::MK;          // MFMA sub-steps per K step
  constexpr int NSUB = kTileN / NMAT;      // output columns per tile
  constexpr int WN = 4 / WM;
  constexpr int TM = BM / WM / 32;         // MFMA tiles per wave along M
  constexpr int TN = kTileN / WN / 32;     // ... along the weight rows
  constexpr int PA = BM / 32;              // 16-byte load passes for A (32 rows each)
  constexpr int P = PA + kTileN / 32;      // passes per K step
  constexpr int NR = TM + TN;              // fragment reads per sub-step
  constexpr int NM = TM * TN;              // MFMAs per sub-step
  constexpr int kStageBytes = (BM + kTileN) * kRowBytes;
  static_assert(NM >= NR, "sub-step pattern assumes at least one MFMA per fragment read");
  __shared__ __align__(16) char lds[2 * kStageBytes];

  // ---- which tile: XCD-contiguous runs, grouped raster inside a run --------
  const int total_m = *g.n_tiles;
  const int NT = g.n_col_tiles;
  const int total = total_m * NT;
  const int b = blockIdx.x;
  if (b >= total) return;
  const int xcd = b & 7, q = total >> 3, rem = total & 7;
  const int l = xcd * q + min(xcd, rem) + (b >> 3);
  const int grp = l / (kGroupM * NT);
  const int gsz = min(kGroupM, total_m - grp * kGroupM);
  const int li = l - grp * kGroupM * NT;
  const int mt = grp * kGroupM + li % gsz;
  const int nt = li / gsz;

  const int s = g.tile_slot[mt];
  const int64_t r0 = g.tile_row0[mt];
  const int64_t rend = min<int64_t>(g.slot_off[s + 1], g.M);
  const int e = g.slot_expert[s];
  if (r0 >= rend || e < 0 || e >= g.E) return;
  const int K = g.K, N = g.N;
  const int n0 = nt * NSUB;
  const int m_valid = static_cast<int>(min<int64_t>(BM, rend - r0));
  const int n_valid = min(NSUB, N - n0);
  const int64_t row_b = static_cast<int64_t>(K) * S;  // bytes per operand row

  const T* A = static_cast<const T*>(g.A) + r0 * K;
  const __amdgpu_buffer_rsrc_t ra = rsrc(A, m_valid * row_b);
  const int64_t wofs = (static_cast<int64_t>(e) * N + n0) * K;
  const __amdgpu_buffer_rsrc_t rb0 = rsrc(static_cast<const T*>(g.B0) + wofs, n_valid * row_b);
  const __amdgpu_buffer_rsrc_t rb1 =
      NMAT > 1 ? rsrc(static_cast<const T*>(g.B1) + wofs, n_valid * row_b) : rb0;

  // ---- global -> register staging: P x 16 bytes per thread per step -------
  // pass p < PA: A rows 32p..; then 8 passes of weight rows (gate/up: 4 + 4)
  const int tid = threadIdx.x;
  const int lrow = tid >> 3, lchunk = tid & 7;
  const int goff = lrow * static_cast<int>(row_b) + lchunk * 16;  // + pass*32 rows + step*128
  const int pass_b = 32 * static_cast<int>(row_b);
  const int loff = lrow * kRowBytes + lchunk * 16;
  uint4 st[P];
  auto issue_one = [&](int p, int o) {
    if (p < PA) st[p] = bload(ra, o + p * pass_b);
    else if (NMAT == 1 || p < PA + 4) st[p] = bload(rb0, o + (p - PA) * pass_b);
    else st[p] = bload(rb1, o + (p - PA - 4) * pass_b);
  };
  auto issue = [&](int kt) {
#pragma unroll
    for (int p = 0; p < P; ++p) issue_one(p, goff + kt * 128);
  };
  auto stash = [&](int stage) {
    char* base = lds + stage * kStageBytes + loff;
#pragma unroll
    for (int p = 0; p < P; ++p) *reinterpret_cast<uint4*>(base + p * 32 * kRowBytes) = st[p];
  };

  // ---- MFMA mapping --------------------------------------------------------
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 31, lg = lane >> 5;
  constexpr int CW = kTileN / WN;  // weight rows per wave
  // weight row (within the tile) of this wave's N-subtile j; with gate and up
  // side by side, subtiles 0 .. TN/2-1 are gate rows, the rest the same up rows
  auto brow = [&](int j) {
    return NMAT == 2 ? (j / (TN / 2)) * 128 + wn * (CW / 2) + (j % (TN / 2)) * 32 : wn * CW + j * 32;
  };
  const int a_rd = (wm * (BM / WM) + lr) * kRowBytes + lg * TR::KV * S;
  int b_rd[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) b_rd[j] = (BM + brow(j) + lr) * kRowBytes + lg * TR::KV * S;

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

  Frag fa[2][TM], fb[2][TN];
  auto frags = [&](const char* sb, int kk, int buf) {
    const int ko = kk * TR::MK * S;
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[buf][i] = *reinterpret_cast<const Frag*>(sb + a_rd + i * 32 * kRowBytes + ko);
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[buf][j] = *reinterpret_cast<const Frag*>(sb + b_rd[j] + ko);
  };
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = mma(fa[buf][i], fb[buf][j], acc[i][j]);
  };

  const int nk = K / BK;
  issue(0);
  stash(0);
  if (nk > 1) issue(1);
  __syncthreads();
  frags(lds, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const char* sb = lds + (kt & 1) * kStageBytes;
    char* wb = lds + ((kt + 1) & 1) * kStageBytes + loff;
    // past the last step the offset is out of range: the loads return zeros
    // without touching memory
    const int o2 = (kt + 2 < nk) ? goff + (kt + 2) * 128 : 0x7ffff000;
    // sub-steps 0 .. KS-2: MFMAs + next fragments + LDS writes of step kt+1 + loads of step kt+2
#pragma unroll
    for (int kk = 0; kk < KS - 1; ++kk) {
      constexpr int PER = (P + KS - 2) / (KS - 1);
      frags(sb, kk + 1, (kk + 1) & 1);
      mfmas(kk & 1);
      int nw = 0;
#pragma unroll
      for (int p = kk * PER; p < (kk + 1) * PER && p < P; ++p) {
        *reinterpret_cast<uint4*>(wb + p * 32 * kRowBytes) = st[p];
        issue_one(p, o2);
        ++nw;
      }
      // interleave: NR x (fragment read, MFMA), then (LDS write, global load,
      // MFMA) while MFMAs last, then the remaining writes/loads and MFMAs
#pragma unroll
      for (int t = 0; t < NR; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
#pragma unroll
      for (int t = 0; t < NM - NR || t < PER; ++t) {
        if (t < nw) {
          __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
        if (t < NM - NR) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    // last sub-step: its fragments are in registers; fetch the next step's first ones
    frags(lds + ((kt + 1) & 1) * kStageBytes, 0, KS & 1);
    mfmas((KS - 1) & 1);
#pragma unroll
    for (int t = 0; t < NR; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- epilogue: lane holds column lr of each 32 x 32 tile, rows
  // 8*(r/4) + 4*lg + r%4 --------------------------------------------------
  T* C = static_cast<T*>(g.C);
  constexpr int JO = NMAT == 2 ? TN / 2 : TN;  // output column subtiles per wave
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < JO; ++j) {
      const int col = n0 + (NMAT == 2 ? wn * (CW / 2) : wn * CW) + j * 32 + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lrow_out = wm * (BM / WM) + i * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
        if (lrow_out >= m_valid || col >= N) continue;
        float v;
        if constexpr (EPI == kEpiSwiGLU) {
          const float gt = acc[i][j][r], up = acc[i][j + TN / 2][r];
          v = gt / (1.f + expf(-gt)) * up;
        } else if constexpr (EPI == kEpiGELU) {
          const float z = acc[i][j][r];
          v = 0.5f * z * (1.f + erff(z * 0.70710678118654752f));
        } else {
          v = acc[i][j][r];
        }
        const int64_t o = (r0 + lrow_out) * N + col;
        if constexpr (kBf16) C[o] = static_cast<uint16_t>(f32_to_bf16_bits(v));
        else C[o] = v;
      }
    }
}

// Lists the row tiles of the GEMMs, per slot s with n rows from `start`:
//   kCover:  ceil(n / BM) tiles from start (the last one may be partial);
//   kPadded: m_pad / BM tiles for every slot with rows, the uniform padded
//            batch (tiles wholly past the slot's last row exit as soon as the
//            GEMM reads them).
enum TileMode { kCover = 0, kPadded = 1 };

__global__ __launch_bounds__(256) void tiles_kernel(const int32_t* __restrict__ slot_off,
                                                    const int32_t* __restrict__ n_slots_p, int max_slots, int64_t M,
                                                    int mode, int BM, int m_pad, int max_tiles,
                                                    int32_t* __restrict__ tile_slot, int32_t* __restrict__ tile_row0,
                                                    int32_t* __restrict__ n_tiles) {
  __shared__ int32_t scan[256];
  __shared__ int32_t carry;
  const int tid = threadIdx.x;
  const int n = min(max(*n_slots_p, 0), max_slots);
  if (tid == 0) carry = 0;
  __syncthreads();
  for (int c = 0; c < n; c += 256) {
    const int s = c + tid;
    int64_t start = 0, cnt = 0;
    if (s < n) {
      start = min<int64_t>(max(slot_off[s], 0), M);
      const int64_t end = min<int64_t>(max(slot_off[s + 1], 0), M);
      const int64_t rows = end > start ? end - start : 0;
      if (mode == kCover) cnt = (rows + BM - 1) / BM;
      else if (rows > 0) cnt = m_pad / BM;
    }
    scan[tid] = static_cast<int32_t>(cnt);
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
      const int32_t v = tid >= d ? scan[tid - d] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    const int32_t first = carry + scan[tid] - static_cast<int32_t>(cnt);
    for (int q = 0; q < cnt; ++q) {
      const int j = first + q;
      if (j < max_tiles) {
        tile_slot[j] = s;
        tile_row0[j] = static_cast<int32_t>(min<int64_t>(start + static_cast<int64_t>(q) * BM, M));
      }
    }
    __syncthreads();
    if (tid == 255) carry += scan[255];
    __syncthreads();
  }
  if (tid == 0) *n_tiles = min(carry, max_tiles);
}

constexpr int kBigM = 256;    // grouped path: 256-row tiles
constexpr int kSmallM = 64;   // dense path: 64-row tiles

struct WsLayout {
  size_t h, tab_slot[2], tab_row0[2], n_tiles, bytes;
  int cap[2];  // tile capacity of each table
};

enum Table { kTabGrouped = 0, kTabPadded = 1 };

// Two tile tables: the grouped 256-row tiles (at most ceil(M/256) + slots) and
// the dense padded batch in 64-row tiles (at most slots x ceil(largest slot /
// 64), the largest slot having at most M rows).
WsLayout ws_layout(moe_dtype dt, int64_t M, int I, int max_slots) {
  WsLayout w{};
  const int64_t cap[2] = {moe::ceil_div(M, kBigM) + max_slots,
                          static_cast<int64_t>(max_slots) * moe::ceil_div(std::max<int64_t>(M, 1), kSmallM)};
  size_t at = 0;
  auto take = [&](size_t n) { size_t p = at; at = moe::align_up(at + n, 256); return p; };
  w.h = take(static_cast<size_t>(M) * I * moe::elem_bytes(dt));
  for (int t = 0; t < 2; ++t) {
    w.cap[t] = static_cast<int>(std::min<int64_t>(cap[t], 0x3fffffff));
    w.tab_slot[t] = take(sizeof(int32_t) * w.cap[t]);
    w.tab_row0[t] = take(sizeof(int32_t) * w.cap[t]);
  }
  w.n_tiles = take(2 * sizeof(int32_t));
  w.bytes = at;
  return w;
}

// Caller-owned events recorded around the two GEMM launches (profiling only).
thread_local hipEvent_t g_timing[3] = {nullptr, nullptr, nullptr};

hipError_t mark(int i, hipStream_t s) { return g_timing[i] ? hipEventRecord(g_timing[i], s) : hipSuccess; }

template <bool kBf16, int EPI, int NMAT>
void launch_gemm(bool dense, const GemmArgs& p, unsigned grid, hipStream_t s) {
  if (dense) gemm_kernel<kBf16, NMAT, EPI, kSmallM, 1><<<grid, 256, 0, s>>>(p);
  else gemm_kernel<kBf16, NMAT, EPI, kBigM, 2><<<grid, 256, 0, s>>>(p);
}

// Phase 1 (gate/up or W1) and phase 2 (down or W2), each on its own tile table.
template <bool kBf16>
int launch_ffn(const GemmArgs& p1, bool dense1, unsigned grid1, const GemmArgs& p2, bool dense2, unsigned grid2,
               bool swiglu, hipStream_t s) {
  if (int rc = moe::hip_status(mark(0, s), "moe_expert_ffn timing event")) return rc;
  if (swiglu) launch_gemm<kBf16, kEpiSwiGLU, 2>(dense1, p1, grid1, s);
  else launch_gemm<kBf16, kEpiGELU, 1>(dense1, p1, grid1, s);
  if (int rc = moe::hip_status(hipGetLastError(), "moe_expert_ffn gate/up launch")) return rc;
  if (int rc = moe::hip_status(mark(1, s), "moe_expert_ffn timing event")) return rc;
  launch_gemm<kBf16, kEpiStore, 1>(dense2, p2, grid2, s);
  if (int rc = moe::hip_status(hipGetLastError(), "moe_expert_ffn down launch")) return rc;
  return moe::hip_status(mark(2, s), "moe_expert_ffn timing event");
}

// AUTO rule, per GEMM: take the dense padded batch when the grouped grid would
// leave more than a quarter of the 256 CUs idle and at most half of the padded
// batch's tiles are padding.
constexpr int kComputeUnits = 256;
bool prefer_dense(int64_t grouped_tiles, int64_t dense_tiles, int64_t dense_real_tiles, int col_tiles) {
  return grouped_tiles * col_tiles * 4 < 3 * kComputeUnits && 2 * dense_real_tiles >= dense_tiles;
}

}  // namespace

extern "C" size_t moe_expert_ffn_workspace_bytes(moe_dtype dt, int64_t M, int H, int I, int max_slots) {
  (void)H;
  if (M < 0 || I < 1 || max_slots < 1 || (dt != MOE_F32 && dt != MOE_BF16)) return 0;
  return ws_layout(dt, M, I, max_slots).bytes;
}

extern "C" int moe_expert_ffn(const void* x_perm, moe_dtype dt, int64_t M, int H, int I, int E,
                              const int32_t* slot_off, const int32_t* slot_expert, const int32_t* n_slots,
                              int max_slots, const void* w_gate, const void* w_up, const void* w_down, moe_act act,
                              moe_gemm_path path, void* y_perm, void* workspace, size_t workspace_bytes,
                              void* stream) {
  using namespace moe;
  if (dt != MOE_F32 && dt != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn: unknown dtype %d", (int)dt);
  if (act != MOE_SWIGLU && act != MOE_GELU) return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn: unknown activation");
  if (path != MOE_GEMM_AUTO && path != MOE_GEMM_GROUPED && path != MOE_GEMM_DENSE)
    return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn: unknown path");
  if (M < 0 || M >= (int64_t(1) << 31)) return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn: M out of range");
  if (H < 64 || I < 64 || H % 64 || I % 64)
    return fail(MOE_ERR_UNSUPPORTED, "moe_expert_ffn: H and I must be positive multiples of 64 (H=%d I=%d)", H, I);
  if (static_cast<int64_t>(std::max(H, I)) * elem_bytes(dt) * kBigM >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "moe_expert_ffn: H or I too large for 32-bit tile offsets");
  if (E < 1 || max_slots < E) return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn: need 1 <= E <= max_slots");
  if (act == MOE_SWIGLU && !w_up) return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn: SwiGLU needs w_up");
  if (act == MOE_GELU && w_up) return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn: GELU takes no w_up (pass NULL)");
  if (!slot_off || !slot_expert || !n_slots || !w_gate || !w_down || !workspace)
    return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn: null pointer");
  if (M > 0 && (!x_perm || !y_perm)) return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn: null pointer");
  for (const void* p : {x_perm, w_gate, w_up, w_down, static_cast<const void*>(y_perm), static_cast<const void*>(workspace)})
    if (p && !aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn: operands must be 16-byte aligned");
  const WsLayout w = ws_layout(dt, M, I, max_slots);
  if (workspace_bytes < w.bytes)
    return fail(MOE_ERR_WORKSPACE, "moe_expert_ffn: workspace has %zu bytes, needs %zu", workspace_bytes, w.bytes);
  if (M == 0) return MOE_OK;

  const hipStream_t s = as_stream(stream);
  const int nt1 = static_cast<int>(ceil_div(I, act == MOE_SWIGLU ? kTileN / 2 : kTileN));
  const int nt2 = static_cast<int>(ceil_div(H, kTileN));
  // GROUPED: 256-row tiles covering each slot.  DENSE: the padded batch in
  // 64-row tiles.  AUTO: per GEMM, from the slot sizes read back here.
  bool dense1 = path == MOE_GEMM_DENSE, dense2 = dense1;
  int m_pad = 0;
  int64_t dense_tiles = 0;
  if (path != MOE_GEMM_GROUPED) {
    std::vector<int32_t> off(static_cast<size_t>(max_slots) + 2);
    if (int rc = hip_status(hipMemcpyAsync(off.data(), slot_off, sizeof(int32_t) * (max_slots + 1),
                                           hipMemcpyDeviceToHost, s), "moe_expert_ffn slot readback")) return rc;
    if (int rc = hip_status(hipMemcpyAsync(&off[max_slots + 1], n_slots, sizeof(int32_t), hipMemcpyDeviceToHost, s),
                            "moe_expert_ffn slot readback")) return rc;
    if (int rc = hip_status(hipStreamSynchronize(s), "moe_expert_ffn slot readback")) return rc;
    const int n = std::min(std::max(off[max_slots + 1], 0), max_slots);
    int64_t largest = 0, active = 0, big_tiles = 0, small_real = 0;
    for (int i = 0; i < n; ++i) {
      const int64_t r = std::max<int64_t>(0, std::min<int64_t>(off[i + 1], M) - std::max<int64_t>(off[i], 0));
      largest = std::max(largest, r);
      if (r > 0) ++active;
      big_tiles += ceil_div(r, kBigM);
      small_real += ceil_div(r, kSmallM);
    }
    m_pad = static_cast<int>(ceil_div(std::max<int64_t>(largest, 1), kSmallM) * kSmallM);
    dense_tiles = active * (m_pad / kSmallM);
    if (path == MOE_GEMM_AUTO) {
      dense1 = prefer_dense(big_tiles, dense_tiles, small_real, nt1);
      dense2 = prefer_dense(big_tiles, dense_tiles, small_real, nt2);
    }
  }
  if ((dense1 || dense2) && dense_tiles > w.cap[kTabPadded])
    return fail(MOE_ERR_WORKSPACE, "moe_expert_ffn: dense path needs %lld tiles", (long long)dense_tiles);

  char* ws = static_cast<char*>(workspace);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(ws + w.n_tiles);
  auto tab_slot = [&](int t) { return reinterpret_cast<int32_t*>(ws + w.tab_slot[t]); };
  auto tab_row0 = [&](int t) { return reinterpret_cast<int32_t*>(ws + w.tab_row0[t]); };
  auto build = [&](int t, int mode, int bm) {
    tiles_kernel<<<1, 256, 0, s>>>(slot_off, n_slots, max_slots, M, mode, bm, m_pad, w.cap[t], tab_slot(t),
                                   tab_row0(t), n_tiles + t);
    return hip_status(hipGetLastError(), "moe_expert_ffn tile-table launch");
  };
  if (!dense1 || !dense2)
    if (int rc = build(kTabGrouped, kCover, kBigM)) return rc;
  if (dense1 || dense2)
    if (int rc = build(kTabPadded, kPadded, kSmallM)) return rc;

  GemmArgs p1{};
  p1.A = x_perm;
  p1.B0 = w_gate;
  p1.B1 = w_up;
  p1.C = ws + w.h;
  p1.M = M;
  p1.K = H;
  p1.N = I;
  p1.E = E;
  p1.slot_off = slot_off;
  p1.slot_expert = slot_expert;
  p1.n_col_tiles = nt1;
  GemmArgs p2 = p1;
  p2.A = ws + w.h;
  p2.B0 = w_down;
  p2.B1 = nullptr;
  p2.C = y_perm;
  p2.K = I;
  p2.N = H;
  p2.n_col_tiles = nt2;
  auto on = [&](GemmArgs& g, bool dense) {
    const int t = dense ? kTabPadded : kTabGrouped;
    g.tile_slot = tab_slot(t);
    g.tile_row0 = tab_row0(t);
    g.n_tiles = n_tiles + t;
  };
  on(p1, dense1);
  on(p2, dense2);
  // grouped: an upper bound on the tiles (blocks past the count exit at once);
  // dense: the exact padded batch
  const int64_t bound = w.cap[kTabGrouped];
  const unsigned grid1 = static_cast<unsigned>(std::max<int64_t>(1, (dense1 ? dense_tiles : bound) * nt1));
  const unsigned grid2 = static_cast<unsigned>(std::max<int64_t>(1, (dense2 ? dense_tiles : bound) * nt2));
  const bool swiglu = act == MOE_SWIGLU;
  return dt == MOE_BF16 ? launch_ffn<true>(p1, dense1, grid1, p2, dense2, grid2, swiglu, s)
                        : launch_ffn<false>(p1, dense1, grid1, p2, dense2, grid2, swiglu, s);
}

extern "C" int moe_ffn_set_timing_events(void* before_gateup, void* after_gateup, void* after_down) {
  const int set = (before_gateup != nullptr) + (after_gateup != nullptr) + (after_down != nullptr);
  if (set != 0 && set != 3) return moe::fail(MOE_ERR_INVALID_ARG, "moe_ffn_set_timing_events: pass three events or none");
  g_timing[0] = static_cast<hipEvent_t>(before_gateup);
  g_timing[1] = static_cast<hipEvent_t>(after_gateup);
  g_timing[2] = static_cast<hipEvent_t>(after_down);
  return MOE_OK;
}
