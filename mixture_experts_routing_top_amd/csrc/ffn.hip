// moe_expert_ffn: the experts' FFNs over the slot-contiguous rows, as grouped
// GEMMs on the MI355X matrix cores.
//
// Source: EPS-MoE review, section 3 (the gate, up and down GEMMs are the
// compute-bound part of an MoE layer; GroupGemm runs every expert's product in
// one kernel; DenseGemm runs a padded uniform batch and wins at small counts).
// SwiGLU h = silu(x Wg^T) * (x Wu^T), y = h Wd^T; GELU h = gelu(x W1^T),
// y = h W2^T.
//
// Two launches of one tiled kernel after a tiny tile-table pass:
//   tiles:   walks the slot table and lists every (slot, 128-row tile) --
//            tiles cover each slot's rows exactly, no host sync.
//   phase 1: for each tile x each block of I columns, the gate and up tiles
//            (or W1) are accumulated side by side so one lane holds g and u of
//            the same element; the activation runs in the epilogue and h is
//            rounded to the dtype once.
//   phase 2: y = h Wd^T over the same tiles, rounded to the dtype.
// 256 threads = 4 waves in 2 x 2; each wave owns a 64 x 64 block per weight
// matrix as 2 x 2 MFMA tiles of 32 x 32 (v_mfma_f32_32x32x16_bf16 for bf16,
// v_mfma_f32_32x32x2f32 for fp32).  A and B tiles are staged through LDS with
// 16-byte global loads, the next K tile prefetched into registers while the
// current one is multiplied.  Each output row depends only on its own input
// row and the fixed K order, so a row's value does not depend on the tile,
// slot or path that computes it.
#include "common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

enum Epi { kEpiSwiGLU = 0, kEpiGELU = 1, kEpiStore = 2 };

template <bool kBf16>
struct Tr;
template <>
struct Tr<true> {
  using T = uint16_t;
  static constexpr int BK = 64;   // K elements per LDS tile (128 bytes per row)
  static constexpr int MK = 16;   // K per MFMA
  static constexpr int KV = 8;    // K elements per lane per MFMA
  static constexpr int PAD = 8;   // row padding (elements) against LDS bank conflicts
  using Frag = uint4;
};
template <>
struct Tr<false> {
  using T = float;
  static constexpr int BK = 32;
  static constexpr int MK = 2;
  static constexpr int KV = 1;
  static constexpr int PAD = 4;
  using Frag = float;
};

__device__ __forceinline__ f32x16 mma(const uint4& a, const uint4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}
__device__ __forceinline__ f32x16 mma(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

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

template <bool kBf16, int BM, int BN, int NMAT, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(GemmArgs g) {
  using TR = Tr<kBf16>;
  using T = typename TR::T;
  using Frag = typename TR::Frag;
  constexpr int BK = TR::BK, LDK = BK + TR::PAD, EPV = 16 / sizeof(T);  // elements per 16 bytes
  constexpr int TM = BM / 64, TN = BN / 64;
  constexpr int PA = BM / 32, PB = BN / 32;  // 16-byte load passes per tile (32 rows per pass)
  __shared__ __align__(16) T As[BM * LDK];
  __shared__ __align__(16) T Bs[NMAT * BN * LDK];

  const int tile = blockIdx.x / g.n_col_tiles;
  const int nt = blockIdx.x - tile * g.n_col_tiles;
  if (tile >= *g.n_tiles) return;
  const int s = g.tile_slot[tile];
  const int64_t r0 = g.tile_row0[tile];
  const int64_t rend = min<int64_t>(g.slot_off[s + 1], g.M);
  const int e = g.slot_expert[s];
  if (r0 >= rend || e < 0 || e >= g.E) return;
  const int n0 = nt * BN;
  const int K = g.K, N = g.N;

  const int tid = threadIdx.x;
  const int lrow = tid >> 3, lchunk = tid & 7;
  const T* A = static_cast<const T*>(g.A);
  const T* Bm[2] = {static_cast<const T*>(g.B0) + static_cast<int64_t>(e) * N * K,
                    NMAT > 1 ? static_cast<const T*>(g.B1) + static_cast<int64_t>(e) * N * K : nullptr};
  const T* a_src[PA];
  const T* b_src[NMAT][PB];
#pragma unroll
  for (int p = 0; p < PA; ++p) {
    const int64_t r = min<int64_t>(r0 + p * 32 + lrow, rend - 1);
    a_src[p] = A + r * K + lchunk * EPV;
  }
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int p = 0; p < PB; ++p) {
      const int64_t n = min(n0 + p * 32 + lrow, N - 1);
      b_src[m][p] = Bm[m] + n * K + lchunk * EPV;
    }

  uint4 ra[PA], rb[NMAT][PB];
  auto load = [&](int kt) {
    const int ko = kt * BK;
#pragma unroll
    for (int p = 0; p < PA; ++p) ra[p] = *reinterpret_cast<const uint4*>(a_src[p] + ko);
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int p = 0; p < PB; ++p) rb[m][p] = *reinterpret_cast<const uint4*>(b_src[m][p] + ko);
  };
  auto stash = [&]() {
#pragma unroll
    for (int p = 0; p < PA; ++p) *reinterpret_cast<uint4*>(&As[(p * 32 + lrow) * LDK + lchunk * EPV]) = ra[p];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int p = 0; p < PB; ++p)
        *reinterpret_cast<uint4*>(&Bs[(m * BN + p * 32 + lrow) * LDK + lchunk * EPV]) = rb[m][p];
  };

  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lg = lane >> 5;
  f32x16 acc[NMAT][TM][TN];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[m][i][j] = f32x16{};

  const int nk = K / BK;
  load(0);
  stash();
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) load(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / TR::MK; ++kk) {
      Frag fa[TM], fb[NMAT][TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        fa[i] = *reinterpret_cast<const Frag*>(&As[(wm * (BM / 2) + i * 32 + lr) * LDK + kk * TR::MK + lg * TR::KV]);
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          fb[m][j] = *reinterpret_cast<const Frag*>(
              &Bs[(m * BN + wn * (BN / 2) + j * 32 + lr) * LDK + kk * TR::MK + lg * TR::KV]);
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) acc[m][i][j] = mma(fa[i], fb[m][j], acc[m][i][j]);
    }
    __syncthreads();
    if (kt + 1 < nk) {
      stash();
      __syncthreads();
    }
  }

  // Epilogue: lane holds column lr of each 32 x 32 tile, rows 8*(r/4) + 4*lg + r%4.
  T* C = static_cast<T*>(g.C);
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * (BN / 2) + j * 32 + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = r0 + wm * (BM / 2) + i * 32 + 8 * (r >> 2) + 4 * lg + (r & 3);
        if (row >= rend || col >= N) continue;
        float v;
        if constexpr (EPI == kEpiSwiGLU) {
          const float gt = acc[0][i][j][r], up = acc[NMAT - 1][i][j][r];
          v = gt / (1.f + expf(-gt)) * up;
        } else if constexpr (EPI == kEpiGELU) {
          const float z = acc[0][i][j][r];
          v = 0.5f * z * (1.f + erff(z * 0.70710678118654752f));
        } else {
          v = acc[0][i][j][r];
        }
        if constexpr (kBf16) C[row * N + col] = static_cast<uint16_t>(f32_to_bf16_bits(v));
        else C[row * N + col] = v;
      }
    }
}

// Lists every (slot, row tile) of the grouped path: tile rows start at the
// slot's first row and step by BM; the last tile of a slot may be partial.
__global__ __launch_bounds__(256) void tiles_kernel(const int32_t* __restrict__ slot_off,
                                                    const int32_t* __restrict__ n_slots_p, int max_slots, int64_t M,
                                                    int BM, int max_tiles, int32_t* __restrict__ tile_slot,
                                                    int32_t* __restrict__ tile_row0, int32_t* __restrict__ n_tiles) {
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
      cnt = end > start ? (end - start + BM - 1) / BM : 0;
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
        tile_row0[j] = static_cast<int32_t>(start + static_cast<int64_t>(q) * BM);
      }
    }
    __syncthreads();
    if (tid == 255) carry += scan[255];
    __syncthreads();
  }
  if (tid == 0) *n_tiles = min(carry, max_tiles);
}

constexpr int kBM = 128, kBN = 128;

struct WsLayout {
  size_t h, tile_slot, tile_row0, n_tiles, bytes;
  int max_tiles;
};

WsLayout ws_layout(moe_dtype dt, int64_t M, int I, int max_slots) {
  WsLayout w{};
  w.max_tiles = static_cast<int>(moe::ceil_div(M, kBM) + max_slots);
  size_t at = 0;
  auto take = [&](size_t n) { size_t p = at; at = moe::align_up(at + n, 256); return p; };
  w.h = take(static_cast<size_t>(M) * I * moe::elem_bytes(dt));
  w.tile_slot = take(sizeof(int32_t) * w.max_tiles);
  w.tile_row0 = take(sizeof(int32_t) * w.max_tiles);
  w.n_tiles = take(sizeof(int32_t));
  w.bytes = at;
  return w;
}

template <bool kBf16>
void launch_ffn(const GemmArgs& p1, const GemmArgs& p2, bool swiglu, unsigned grid1, unsigned grid2, hipStream_t s) {
  if (swiglu) gemm_kernel<kBf16, kBM, kBN, 2, kEpiSwiGLU><<<grid1, 256, 0, s>>>(p1);
  else gemm_kernel<kBf16, kBM, kBN, 1, kEpiGELU><<<grid1, 256, 0, s>>>(p1);
  gemm_kernel<kBf16, kBM, kBN, 1, kEpiStore><<<grid2, 256, 0, s>>>(p2);
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
  char* ws = static_cast<char*>(workspace);
  int32_t* tile_slot = reinterpret_cast<int32_t*>(ws + w.tile_slot);
  int32_t* tile_row0 = reinterpret_cast<int32_t*>(ws + w.tile_row0);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(ws + w.n_tiles);
  tiles_kernel<<<1, 256, 0, s>>>(slot_off, n_slots, max_slots, M, kBM, w.max_tiles, tile_slot, tile_row0, n_tiles);

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
  p1.tile_slot = tile_slot;
  p1.tile_row0 = tile_row0;
  p1.n_tiles = n_tiles;
  p1.n_col_tiles = static_cast<int>(ceil_div(I, kBN));
  GemmArgs p2 = p1;
  p2.A = ws + w.h;
  p2.B0 = w_down;
  p2.B1 = nullptr;
  p2.C = y_perm;
  p2.K = I;
  p2.N = H;
  p2.n_col_tiles = static_cast<int>(ceil_div(H, kBN));
  const unsigned grid1 = static_cast<unsigned>(w.max_tiles) * p1.n_col_tiles;
  const unsigned grid2 = static_cast<unsigned>(w.max_tiles) * p2.n_col_tiles;
  if (dt == MOE_BF16) launch_ffn<true>(p1, p2, act == MOE_SWIGLU, grid1, grid2, s);
  else launch_ffn<false>(p1, p2, act == MOE_SWIGLU, grid1, grid2, s);
  return hip_status(hipGetLastError(), "moe_expert_ffn launch");
}
