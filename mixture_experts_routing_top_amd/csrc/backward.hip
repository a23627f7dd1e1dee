// moe_backward: gradients of one MoE layer's forward pass w.r.t. its input
// tokens, its router logits and its expert weights, given d_out.
//
// Sources: PopFetcher wiki, method (MoE training: the backward pass follows
// the forward, with its own All-to-All in the opposite direction); the
// expert-load prediction study (training iterations); EPS-MoE review, section
// 3 (the expert GEMMs are the compute-bound part; GroupGemm per expert).  The
// gradients themselves are the chain rule through the forward's definition.
//
// Stream-ordered steps (M = T*k rows in expert-contiguous order, as dispatched):
//   1. gate + combine transpose, one block per token: dw[t,i] = <d_out[t],
//      y_perm[r]>, d_y[r] = w[t,i] d_out[t] for r = inv_pos[t,i], and the
//      softmax Jacobian over the kept logits, d_l[t,e_j] = w_j (dw_j - sum_i
//      w_i dw_i) (zero for the other experts);
//   2. d_h = d_y Wd by the grouped GEMM, kept in fp32 [M, I];
//   3. the gate/up (or W1) pre-activations recomputed by the grouped GEMM
//      (activation recomputation rather than a saved [M, 2I]); its epilogue
//      meets their fp32 accumulators with d_h: the activation gradient
//      d_g | d_u (or d_z) and h, rebuilt with the forward's own activation so
//      it rounds as the forward rounded it, both in the dtype;
//   4. weight gradient of Wd: one expert-grouped GEMM whose K range is each
//      expert's rows of d_y and h;
//   5. d_x_perm = d_g Wg + d_u Wu as one GEMM with K = 2I over [Wg; Wu];
//   6. d_x = the unweighted sum of each token's k rows (the combine kernel);
//   7. weight gradients of Wg, Wu (or W1) from d_g | d_u and x_perm, the same
//      way.
// Steps 2, 4, 5 and 7 contract over a dimension that is not contiguous in
// memory (the weights' rows, the activations' rows).  bf16 tiles read those
// operands in place, K-major, through the transposed LDS read (gemm.h); fp32
// tiles take K-contiguous operands only, so for fp32 the weights are
// transposed first and the activations transposed into per-expert K ranges
// padded to the K step.
#include <algorithm>

#include "common.h"
#include "gemm.h"

namespace {

constexpr int kTok = 256;  // threads per token block in step 1

// Step 1.  Thread tid handles 16-byte chunks tid, tid + 256, ... of the row.
template <bool kBf16>
__global__ __launch_bounds__(kTok) void gate_backward_kernel(const uint4* __restrict__ d_out,
                                                             const uint4* __restrict__ y_perm, int64_t M,
                                                             const int32_t* __restrict__ topk_idx,
                                                             const float* __restrict__ topk_w,
                                                             const int32_t* __restrict__ inv_pos, int k, int E,
                                                             int chunks, uint4* __restrict__ d_y,
                                                             float* __restrict__ d_logits) {
  __shared__ float part[kTok / 64][moe::kMaxTopK];
  __shared__ float dw[moe::kMaxTopK];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  int32_t rows[moe::kMaxTopK];
  float wi[moe::kMaxTopK], acc[moe::kMaxTopK];
#pragma unroll
  for (int i = 0; i < moe::kMaxTopK; ++i) {
    rows[i] = -1;
    wi[i] = 0.f;
    acc[i] = 0.f;
    if (i < k) {
      const int32_t r = inv_pos[t * k + i];
      rows[i] = (r >= 0 && r < M) ? r : -1;
      wi[i] = topk_w[t * k + i];
    }
  }
  constexpr int V = kBf16 ? 8 : 4;
  for (int c = tid; c < chunks; c += kTok) {
    const uint4 q = d_out[t * chunks + c];
    const uint32_t qv[4] = {q.x, q.y, q.z, q.w};
    float o[V];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (kBf16) {
        o[2 * j] = bf16_bits_to_f32(qv[j] & 0xffffu);
        o[2 * j + 1] = bf16_bits_to_f32(qv[j] >> 16);
      } else {
        o[j] = __uint_as_float(qv[j]);
      }
    }
#pragma unroll
    for (int i = 0; i < moe::kMaxTopK; ++i) {
      if (i >= k || rows[i] < 0) continue;
      const uint4 yq = y_perm[static_cast<int64_t>(rows[i]) * chunks + c];
      const uint32_t yv[4] = {yq.x, yq.y, yq.z, yq.w};
      uint32_t dv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (kBf16) {
          acc[i] = fmaf(o[2 * j], bf16_bits_to_f32(yv[j] & 0xffffu), acc[i]);
          acc[i] = fmaf(o[2 * j + 1], bf16_bits_to_f32(yv[j] >> 16), acc[i]);
          dv[j] = f32_to_bf16_bits(wi[i] * o[2 * j]) | (f32_to_bf16_bits(wi[i] * o[2 * j + 1]) << 16);
        } else {
          acc[i] = fmaf(o[j], __uint_as_float(yv[j]), acc[i]);
          dv[j] = __float_as_uint(wi[i] * o[j]);
        }
      }
      d_y[static_cast<int64_t>(rows[i]) * chunks + c] = make_uint4(dv[0], dv[1], dv[2], dv[3]);
    }
  }
  // block reduction of the k dot products, in a fixed order
  const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
  for (int i = 0; i < moe::kMaxTopK; ++i) {
    if (i >= k) break;
    float v = acc[i];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0) part[wave][i] = v;
  }
  __syncthreads();
  if (tid < k) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kTok / 64; ++w) v += part[w][tid];
    dw[tid] = v;
  }
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < k; ++i) s = fmaf(wi[i], dw[i], s);
  for (int e = tid; e < E; e += kTok) {
    float v = 0.f;
    for (int i = 0; i < k; ++i)
      if (topk_idx[t * k + i] == e && rows[i] >= 0) v = wi[i] * (dw[i] - s);
    d_logits[t * E + e] = v;
  }
}

// dst[b][c][col_off + r] = src[b][r][c] for a batch of R x C matrices; dst rows
// are ld elements long.  64 x 64 tiles through LDS, 16-byte global accesses
// (R, C, ld and col_off are multiples of 64).
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, int R, int C, T* __restrict__ dst,
                                                        int ld, int col_off) {
  constexpr int V = 16 / sizeof(T);   // elements per 16-byte chunk
  constexpr int CH = 64 / V;          // chunks per 64-element row
  __shared__ T tile[64][64 + 2];
  const int b = blockIdx.z;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const T* s = src + static_cast<int64_t>(b) * R * C;
  T* d = dst + static_cast<int64_t>(b) * C * ld;
  for (int q = threadIdx.x; q < 64 * CH; q += 256) {
    const int y = q / CH, x = (q % CH) * V;
    const uint4 v = *reinterpret_cast<const uint4*>(s + static_cast<int64_t>(r0 + y) * C + c0 + x);
    const T* e = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int u = 0; u < V; ++u) tile[y][x + u] = e[u];
  }
  __syncthreads();
  for (int q = threadIdx.x; q < 64 * CH; q += 256) {
    const int y = q / CH, x = (q % CH) * V;   // destination row c0 + y, columns r0 + x ..
    uint4 v;
    T* e = reinterpret_cast<T*>(&v);
#pragma unroll
    for (int u = 0; u < V; ++u) e[u] = tile[x + u][y];
    *reinterpret_cast<uint4*>(d + static_cast<int64_t>(c0 + y) * ld + col_off + r0 + x) = v;
  }
}

// Expert-padded transpose of row-major [M, C] activations into [C, ld]: expert
// e's rows off[e] .. off[e+1] become columns seg[e] .. (zero to seg[e+1]).
// Column blocks of 64 never straddle experts (segments are multiples of 64); C
// is a multiple of 64.  64 x 64 tiles through LDS with 16-byte global loads and
// stores.
template <bool kBf16>
__global__ __launch_bounds__(256) void transpose_padded_kernel(const void* __restrict__ src, int64_t M, int C,
                                                               const int32_t* __restrict__ off,
                                                               const int32_t* __restrict__ seg, int E,
                                                               void* __restrict__ dst, int ld) {
  using T = typename Tr<kBf16>::T;
  constexpr int V = 16 / sizeof(T);  // elements per 16-byte access
  __shared__ T tile[64][64 + 2];
  const int j0 = blockIdx.y * 64;  // destination column block (padded row index)
  const int c0 = blockIdx.x * 64;  // source column block
  if (j0 >= seg[E]) return;
  int e = 0;
  while (e + 1 < E && seg[e + 1] <= j0) ++e;
  const int64_t n_e = min<int64_t>(static_cast<int64_t>(off[e + 1]) - off[e], seg[e + 1] - seg[e]);
  const int64_t base = off[e] + (j0 - seg[e]);
  for (int q = threadIdx.x; q < 64 * (64 / V); q += 256) {
    const int y = q / (64 / V), x = (q % (64 / V)) * V;  // source row base + y, columns c0 + x ..
    const int64_t row = base + y;
    const bool ok = (j0 - seg[e]) + y < n_e && row >= 0 && row < M;
    const uint4 raw = ok ? *reinterpret_cast<const uint4*>(static_cast<const T*>(src) + row * C + c0 + x)
                         : make_uint4(0, 0, 0, 0);
    T v[V];
    __builtin_memcpy(v, &raw, sizeof(raw));
#pragma unroll
    for (int u = 0; u < V; ++u) tile[y][x + u] = v[u];
  }
  __syncthreads();
  T* d = static_cast<T*>(dst);
  for (int q = threadIdx.x; q < 64 * (64 / V); q += 256) {
    const int y = q / (64 / V), x = (q % (64 / V)) * V;  // destination row c0 + y, columns j0 + x ..
    T v[V];
#pragma unroll
    for (int u = 0; u < V; ++u) v[u] = tile[x + u][y];
    uint4 raw;
    __builtin_memcpy(&raw, v, sizeof(raw));
    *reinterpret_cast<uint4*>(d + static_cast<int64_t>(c0 + y) * ld + j0 + x) = raw;
  }
}

// seg[e] = sum over e' < e of n_e' rounded up to 64 (n_e clamped to [0, M], the
// sum to the transposed row length ld, so malformed offsets cannot reach past
// the buffers); slot table = experts; ones.
__global__ void bwd_setup_kernel(const int32_t* __restrict__ off, int E, int64_t M, int64_t ld,
                                 int32_t* __restrict__ seg, int32_t* __restrict__ slot_expert,
                                 int32_t* __restrict__ n_slots, float* __restrict__ ones, int64_t n_ones) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    int64_t s = 0;
    for (int e = 0; e < E; ++e) {
      seg[e] = static_cast<int32_t>(s);
      const int64_t n = min<int64_t>(max<int64_t>(static_cast<int64_t>(off[e + 1]) - off[e], 0), M);
      s = min<int64_t>(s + (n + 63) / 64 * 64, ld / 64 * 64);
    }
    seg[E] = static_cast<int32_t>(s);
    *n_slots = E;
  }
  for (int e = tid; e < E; e += blockDim.x) slot_expert[e] = e;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + tid; i < n_ones;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    ones[i] = 1.f;
}

// blocks of a weight-gradient launch: 8 equal shares of each expert's
// (256-row x 256-column) tiles
unsigned wgrad_grid(int E, int64_t rows, int col_tiles) {
  const int64_t per_e = moe::ceil_div(rows, 256) * col_tiles;
  return static_cast<unsigned>(8 * E * moe::ceil_div(per_e, 8));
}

struct BwdLayout {
  size_t dh, h, dgu, dy, wdT, wguT, ta, tb, ones, seg, slot_expert, n_slots, tab_slot, tab_row0, tab_rend, n_tiles,
      bytes;
  int64_t ld;  // padded row length of the transposed activations
  int tiles_cap;
};

BwdLayout bwd_layout(moe_dtype dt, int64_t T, int k, int H, int I, int E, moe_act act) {
  BwdLayout w{};
  const size_t s = moe::elem_bytes(dt);
  const bool tr = dt != MOE_BF16;  // transposed copies (fp32 only)
  const int64_t M = T * k;
  const int64_t nI = act == MOE_SWIGLU ? 2 * static_cast<int64_t>(I) : I;  // gate|up columns
  w.ld = moe::ceil_div(M, 64) * 64 + 64 * static_cast<int64_t>(E);
  w.tiles_cap = static_cast<int>(moe::ceil_div(M, 256) + E);
  size_t at = 0;
  auto take = [&](size_t n) { size_t p = at; at = moe::align_up(at + n, 256); return p; };
  w.dh = take(static_cast<size_t>(M) * I * 4);
  w.h = take(static_cast<size_t>(M) * I * s);
  w.dgu = take(static_cast<size_t>(M) * nI * s);
  w.dy = take(static_cast<size_t>(M) * H * s);
  w.wdT = take(tr ? static_cast<size_t>(E) * I * H * s : 0);
  w.wguT = take(tr ? static_cast<size_t>(E) * H * nI * s : 0);
  w.ta = take(tr ? static_cast<size_t>(std::max<int64_t>(H, nI)) * w.ld * s : 0);
  w.tb = take(tr ? static_cast<size_t>(std::max<int64_t>(I, H)) * w.ld * s : 0);
  w.ones = take(static_cast<size_t>(M) * 4);
  w.seg = take(sizeof(int32_t) * (E + 1));
  w.slot_expert = take(sizeof(int32_t) * E);
  w.n_slots = take(sizeof(int32_t));
  w.tab_slot = take(sizeof(int32_t) * w.tiles_cap);
  w.tab_row0 = take(sizeof(int32_t) * w.tiles_cap);
  w.tab_rend = take(sizeof(int32_t) * w.tiles_cap);
  w.n_tiles = take(sizeof(int32_t));
  w.bytes = at;
  return w;
}

template <bool kBf16>
int run_backward(const void* x_perm, const void* y_perm, int64_t n_tok, int k, int H, int I, int E,
                 const int32_t* topk_idx, const float* topk_w, const int32_t* inv_pos, const int32_t* expert_off,
                 const void* w_gate, const void* w_up, const void* w_down, bool swiglu, const void* d_out,
                 void* d_x, float* d_logits, void* d_w_gate, void* d_w_up, void* d_w_down, char* ws,
                 const BwdLayout& L, hipStream_t s) {
  using namespace moe;
  using T = typename Tr<kBf16>::T;
  const int64_t M = n_tok * k;
  const int S = sizeof(T);
  const int nI = swiglu ? 2 * I : I;
  auto at = [&](size_t o) { return ws + o; };
  float* dh = reinterpret_cast<float*>(at(L.dh));
  T* hbuf = reinterpret_cast<T*>(at(L.h));
  T* dgu = reinterpret_cast<T*>(at(L.dgu));
  T* dy = reinterpret_cast<T*>(at(L.dy));
  T* wdT = reinterpret_cast<T*>(at(L.wdT));
  T* wguT = reinterpret_cast<T*>(at(L.wguT));
  T* ta = reinterpret_cast<T*>(at(L.ta));
  T* tb = reinterpret_cast<T*>(at(L.tb));
  float* ones = reinterpret_cast<float*>(at(L.ones));
  int32_t* seg = reinterpret_cast<int32_t*>(at(L.seg));
  int32_t* slot_expert = reinterpret_cast<int32_t*>(at(L.slot_expert));
  int32_t* n_slots = reinterpret_cast<int32_t*>(at(L.n_slots));
  int32_t* tab_slot = reinterpret_cast<int32_t*>(at(L.tab_slot));
  int32_t* tab_row0 = reinterpret_cast<int32_t*>(at(L.tab_row0));
  int32_t* tab_rend = reinterpret_cast<int32_t*>(at(L.tab_rend));
  int32_t* n_tiles = reinterpret_cast<int32_t*>(at(L.n_tiles));
  auto check = [&](const char* what) { return hip_status(hipGetLastError(), what); };

  bwd_setup_kernel<<<static_cast<unsigned>(std::min<int64_t>(1024, ceil_div(M, 256)) + 1), 256, 0, s>>>(
      expert_off, E, M, L.ld, seg, slot_expert, n_slots, ones, M);
  tiles_kernel<<<1, 256, 0, s>>>(expert_off, slot_expert, n_slots, E, M, E, kCover, 256, 0, 0, L.tiles_cap, tab_slot,
                                 tab_row0, tab_rend, n_tiles, TileSplit{}, nullptr);
  if (int rc = check("moe_backward setup")) return rc;

  // 1. gate + combine transpose
  const int chunks = static_cast<int>(static_cast<int64_t>(H) * S / 16);
  if (n_tok > 0)
    gate_backward_kernel<kBf16><<<static_cast<unsigned>(n_tok), kTok, 0, s>>>(
        static_cast<const uint4*>(d_out), static_cast<const uint4*>(y_perm), M, topk_idx, topk_w, inv_pos, k, E,
        chunks, reinterpret_cast<uint4*>(dy), d_logits);
  if (int rc = check("moe_backward gate")) return rc;

  // fp32: transposed weights WdT [E, I, H]; WguT [E, H, 2I] = [Wg^T | Wu^T] (or W1^T [E, H, I])
  if constexpr (!kBf16) {
    const dim3 tb_d(ceil_div(I, 64), ceil_div(H, 64), E), tb_g(ceil_div(H, 64), ceil_div(I, 64), E);
    transpose_kernel<T><<<tb_d, 256, 0, s>>>(static_cast<const T*>(w_down), H, I, wdT, H, 0);
    transpose_kernel<T><<<tb_g, 256, 0, s>>>(static_cast<const T*>(w_gate), I, H, wguT, nI, 0);
    if (swiglu) transpose_kernel<T><<<tb_g, 256, 0, s>>>(static_cast<const T*>(w_up), I, H, wguT, nI, I);
    if (int rc = check("moe_backward weight transposes")) return rc;
  }

  GemmArgs base{};
  base.M = M;
  base.E = E;
  base.slot_off = expert_off;
  base.slot_expert = slot_expert;
  base.tile_slot = tab_slot;
  base.tile_row0 = tab_row0;
  base.tile_rend = tab_rend;
  base.n_tiles = n_tiles;
  const unsigned grid_rows = static_cast<unsigned>(L.tiles_cap);

  // 2. d_h = d_y Wd in fp32 (bf16: Wd [E, H, I] read K-major)
  GemmArgs p = base;
  p.A = dy;
  p.B0 = kBf16 ? w_down : wdT;
  p.ldb = I;
  p.C = dh;
  p.K = H;
  p.N = I;
  p.n_col_tiles = static_cast<int>(ceil_div(I, kTileN));
  if constexpr (kBf16)
    gemm_kernel<kBf16, 1, kEpiStoreF32, 256, 2, false, 2><<<grid_rows * p.n_col_tiles, 256, 0, s>>>(p);
  else
    gemm_kernel<kBf16, 1, kEpiStoreF32, 256, 2><<<grid_rows * p.n_col_tiles, 256, 0, s>>>(p);
  if (int rc = check("moe_backward d_h")) return rc;

  // 3. recompute the pre-activations; the epilogue turns d_h into d_g | d_u
  //    (or d_z) and rebuilds h
  p = base;
  p.A = x_perm;
  p.B0 = w_gate;
  p.B1 = w_up;
  p.C = dgu;
  p.C2 = hbuf;
  p.aux = dh;
  p.K = H;
  p.N = I;
  if (swiglu) {
    p.n_col_tiles = static_cast<int>(ceil_div(I, kTileN / 2));
    gemm_kernel<kBf16, 2, kEpiSwiGLUGrad, 256, 2><<<grid_rows * p.n_col_tiles, 256, 0, s>>>(p);
  } else {
    p.n_col_tiles = static_cast<int>(ceil_div(I, kTileN));
    gemm_kernel<kBf16, 1, kEpiGELUGrad, 256, 2><<<grid_rows * p.n_col_tiles, 256, 0, s>>>(p);
  }
  if (int rc = check("moe_backward recompute")) return rc;

  // 4. d_Wd = sum over each expert's rows of d_y^T h (bf16: d_y [M, H] and h
  //    [M, I] read K-major in place; fp32: both transposed into padded K ranges)
  const int ld = static_cast<int>(L.ld);
  const unsigned ldb = static_cast<unsigned>(ceil_div(L.ld, 64));
  GemmArgs q{};
  q.C = d_w_down;
  q.C2 = d_w_down;
  q.M = M;
  q.E = E;
  q.N = I;
  q.Mw = H;
  q.c_split = H;
  q.n_col_tiles = static_cast<int>(ceil_div(I, kTileN));
  if constexpr (kBf16) {
    q.A = dy;
    q.lda = H;
    q.B0 = hbuf;
    q.ldb = I;
    q.slot_off = expert_off;
    gemm_kernel<kBf16, 1, kEpiStore, 256, 2, true, 3><<<wgrad_grid(E, H, q.n_col_tiles), 256, 0, s>>>(q);
  } else {
    transpose_padded_kernel<kBf16><<<dim3(ceil_div(H, 64), ldb), 256, 0, s>>>(dy, M, H, expert_off, seg, E, ta,
                                                                                    ld);
    transpose_padded_kernel<kBf16><<<dim3(ceil_div(I, 64), ldb), 256, 0, s>>>(hbuf, M, I, expert_off, seg, E,
                                                                                    tb, ld);
    q.A = ta;
    q.B0 = tb;
    q.ld = ld;
    q.seg = seg;
    gemm_kernel<kBf16, 1, kEpiStore, 256, 2, true><<<wgrad_grid(E, H, q.n_col_tiles), 256, 0, s>>>(q);
  }
  if (int rc = check("moe_backward d_Wd")) return rc;

  // 5. d_x_perm = [d_g | d_u] [Wg ; Wu] (into the d_y buffer, no longer needed;
  //    bf16: Wg and Wu [E, I, H] read K-major, K rows from Wg then Wu)
  p = base;
  p.A = dgu;
  p.C = dy;
  p.K = nI;
  p.N = H;
  p.n_col_tiles = static_cast<int>(ceil_div(H, kTileN));
  if constexpr (kBf16) {
    p.B0 = w_gate;
    p.B1 = swiglu ? w_up : nullptr;
    p.k_split = swiglu ? I : 0;
    p.ldb = H;
    gemm_kernel<kBf16, 1, kEpiStore, 256, 2, false, 2><<<grid_rows * p.n_col_tiles, 256, 0, s>>>(p);
  } else {
    p.B0 = wguT;
    gemm_kernel<kBf16, 1, kEpiStore, 256, 2><<<grid_rows * p.n_col_tiles, 256, 0, s>>>(p);
  }
  if (int rc = check("moe_backward d_x_perm")) return rc;

  // 6. d_x[t] = sum of the token's k rows
  if (int rc = moe_combine(dy, kBf16 ? MOE_BF16 : MOE_F32, M, inv_pos, ones, n_tok, k, H, d_x, nullptr, s)) return rc;

  // 7. d_Wg | d_Wu (or d_W1) = sum over each expert's rows of [d_g | d_u]^T x_perm
  q.C = d_w_gate;
  q.C2 = swiglu ? d_w_up : d_w_gate;
  q.N = H;
  q.Mw = nI;
  q.c_split = I;
  q.n_col_tiles = static_cast<int>(ceil_div(H, kTileN));
  if constexpr (kBf16) {
    q.A = dgu;
    q.lda = nI;
    q.B0 = x_perm;
    q.ldb = H;
    gemm_kernel<kBf16, 1, kEpiStore, 256, 2, true, 3><<<wgrad_grid(E, nI, q.n_col_tiles), 256, 0, s>>>(q);
  } else {
    transpose_padded_kernel<kBf16><<<dim3(ceil_div(nI, 64), ldb), 256, 0, s>>>(dgu, M, nI, expert_off, seg, E,
                                                                                     ta, ld);
    transpose_padded_kernel<kBf16><<<dim3(ceil_div(H, 64), ldb), 256, 0, s>>>(x_perm, M, H, expert_off, seg, E,
                                                                                    tb, ld);
    q.A = ta;
    q.B0 = tb;
    gemm_kernel<kBf16, 1, kEpiStore, 256, 2, true><<<wgrad_grid(E, nI, q.n_col_tiles), 256, 0, s>>>(q);
  }
  return check("moe_backward d_Wg/d_Wu");
}

}  // namespace

extern "C" size_t moe_backward_workspace_bytes(moe_dtype dt, int64_t T, int k, int H, int I, int E, moe_act act) {
  if (T < 0 || k < 1 || H < 1 || I < 1 || E < 1 || (dt != MOE_F32 && dt != MOE_BF16)) return 0;
  return bwd_layout(dt, T, k, H, I, E, act).bytes;
}

extern "C" int moe_backward(const void* x_perm, const void* y_perm, moe_dtype dt, int64_t T, int k, int H, int I,
                            int E, const int32_t* topk_idx, const float* topk_w, const int32_t* inv_pos,
                            const int32_t* expert_off, const void* w_gate, const void* w_up, const void* w_down,
                            moe_act act, const void* d_out, void* d_x, float* d_logits, void* d_w_gate,
                            void* d_w_up, void* d_w_down, void* workspace, size_t workspace_bytes, void* stream) {
  using namespace moe;
  if (dt != MOE_F32 && dt != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "moe_backward: unknown dtype %d", (int)dt);
  if (act != MOE_SWIGLU && act != MOE_GELU) return fail(MOE_ERR_INVALID_ARG, "moe_backward: unknown activation");
  if (E < 1 || E > kMaxExperts)
    return fail(E < 1 ? MOE_ERR_INVALID_ARG : MOE_ERR_UNSUPPORTED, "moe_backward: E=%d outside [1, %d]", E,
                kMaxExperts);
  if (k < 1 || k > E || k > kMaxTopK) return fail(MOE_ERR_INVALID_ARG, "moe_backward: k=%d outside [1, min(E, 8)]", k);
  if (T < 0 || T * k >= (int64_t(1) << 30)) return fail(MOE_ERR_INVALID_ARG, "moe_backward: T*k must stay below 2^30");
  if (H < 64 || I < 64 || H % 64 || I % 64)
    return fail(MOE_ERR_UNSUPPORTED, "moe_backward: H and I must be positive multiples of 64 (H=%d I=%d)", H, I);
  const int nI = act == MOE_SWIGLU ? 2 * I : I;
  const BwdLayout L = bwd_layout(dt, T, k, H, I, E, act);
  if (static_cast<int64_t>(std::max(H, nI)) * elem_bytes(dt) * 256 >= (int64_t(1) << 31) ||
      L.ld * elem_bytes(dt) * 256 >= (int64_t(1) << 31))
    return fail(MOE_ERR_UNSUPPORTED, "moe_backward: sizes too large for 32-bit tile offsets");
  {
    // block and tile indices are 32-bit in the kernels: bound every GEMM grid
    // (at most 128 output columns per column tile)
    const int64_t wide = std::max<int64_t>(H, nI);
    const int64_t max_nt = ceil_div(wide, 128);
    const int64_t rows_grid = static_cast<int64_t>(L.tiles_cap) * max_nt;
    const int64_t wgrad_blocks = static_cast<int64_t>(E) * (ceil_div(wide, 256) * max_nt + 8);
    if (std::max(rows_grid, wgrad_blocks) >= (int64_t(1) << 31) - 256)
      return fail(MOE_ERR_UNSUPPORTED, "moe_backward: sizes exceed 32-bit grid indexing");
  }
  if (act == MOE_SWIGLU && !w_up) return fail(MOE_ERR_INVALID_ARG, "moe_backward: SwiGLU needs w_up");
  if (act == MOE_GELU && (w_up || d_w_up)) return fail(MOE_ERR_INVALID_ARG, "moe_backward: GELU takes no w_up/d_w_up");
  if (!expert_off || !w_gate || !w_down || !d_w_gate || !d_w_down || !workspace || (act == MOE_SWIGLU && !d_w_up))
    return fail(MOE_ERR_INVALID_ARG, "moe_backward: null pointer");
  if (T > 0 && (!x_perm || !y_perm || !topk_idx || !topk_w || !inv_pos || !d_out || !d_x || !d_logits))
    return fail(MOE_ERR_INVALID_ARG, "moe_backward: null pointer");
  const void* ptrs[] = {x_perm, y_perm, w_gate, w_up, w_down, d_out, d_x, d_w_gate, d_w_up, d_w_down, workspace};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "moe_backward: operands must be 16-byte aligned");
  if (workspace_bytes < L.bytes)
    return fail(MOE_ERR_WORKSPACE, "moe_backward: workspace has %zu bytes, needs %zu", workspace_bytes, L.bytes);
  const hipStream_t s = as_stream(stream);
  char* ws = static_cast<char*>(workspace);
  return dt == MOE_BF16
             ? run_backward<true>(x_perm, y_perm, T, k, H, I, E, topk_idx, topk_w, inv_pos, expert_off, w_gate, w_up,
                                  w_down, act == MOE_SWIGLU, d_out, d_x, d_logits, d_w_gate, d_w_up, d_w_down, ws, L, s)
             : run_backward<false>(x_perm, y_perm, T, k, H, I, E, topk_idx, topk_w, inv_pos, expert_off, w_gate,
                                   w_up, w_down, act == MOE_SWIGLU, d_out, d_x, d_logits, d_w_gate, d_w_up, d_w_down,
                                   ws, L, s);
}
