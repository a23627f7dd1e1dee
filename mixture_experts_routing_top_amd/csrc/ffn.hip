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
#include "gemm.h"

namespace {

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
