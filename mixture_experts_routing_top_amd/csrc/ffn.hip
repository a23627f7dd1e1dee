// moe_expert_ffn: the experts' FFNs over the slot-contiguous rows, as grouped
// GEMMs on the MI355X matrix cores.
//
// Source: EPS-MoE review, section 3 (the gate, up and down GEMMs are the
// compute-bound part of an MoE layer; GroupGemm runs every expert's product in
// one kernel; DenseGemm runs a padded uniform batch and wins at small counts).
// SwiGLU h = silu(x Wg^T) * (x Wu^T), y = h Wd^T; GELU h = gelu(x W1^T),
// y = h W2^T.
//
// A tile-table pass, then two launches of the tiled MFMA kernel of gemm.h:
//   tiles:   lists the row tiles of a GEMM: 256-row tiles covering each slot
//            (GROUPED; a range of <= 64 rows and, when the launch's last
//            round would be mostly idle, the trailing row tiles go to a 64-row
//            companion table run by the same launch), 64-row tiles covering
//            each slot (GROUPED_SMALL), or every active slot padded to the
//            largest (DENSE); AUTO reads the slot sizes back and picks per
//            GEMM by a fitted cost model.
//   phase 1: per tile and per 128 columns of I, the gate and up weight tiles
//            are multiplied side by side so one lane holds g and u of the same
//            element; the activation runs in the epilogue and h is rounded to
//            the dtype once (GELU: one 256-column weight tile).
//   phase 2: y = h Wd^T per tile and 256 columns of H, rounded to the dtype.
// Each output row depends only on its own input row and the fixed K order, so
// a row's value does not depend on the tile, slot or path that computes it.
#include <algorithm>
#include <vector>

#include "common.h"
#include "gemm.h"

namespace {

constexpr int kBigM = 256;    // grouped path: 256-row tiles
constexpr int kSmallM = 64;   // dense path: 64-row tiles

struct WsLayout {
  size_t h, tab_slot[3], tab_row0[3], tab_rend[3], n_tiles, split_slot, split_row0, split_rend, split_counts,
      mid_slot, mid_row0, mid_rend, alt_slot, alt_row0, alt_rend, steal, bytes;
  int cap[3];     // tile capacity of each table
  int split_cap;  // entries of each GEMM's 64-row companion table
};

// AUTO's cost of a 64-row tile in 256-row tiles (see pick_kind), and the most
// 64-row tiles a short range may take in a 256-row tiling: while they cost
// less than one 256-row tile (1 at 0.55, i.e. ranges of <= 64 rows).
constexpr double kSmallCost = 0.55;
constexpr int kRemTiles = kSmallCost >= 0.5 ? 1 : kSmallCost >= 1.0 / 3 ? 2 : 3;
// 64-row tiles re-listing a 256-row table's trailing row tiles: at most
// ceil(256 / column tiles) of them, four each.
constexpr int kConvCap = 4 * 256;

// The row tilings a GEMM can run on, each with its own tile table:
//   kG256: 256-row tiles covering each slot (at most ceil(M/256) + slots);
//   kD64:  the dense padded batch in 64-row tiles (at most slots x ceil(M/64));
//   kG64:  64-row tiles covering each slot (at most ceil(M/64) + slots).
enum Kind { kG256 = 0, kD64 = 1, kG64 = 2 };

WsLayout ws_layout(moe_dtype dt, int64_t M, int I, int max_slots) {
  WsLayout w{};
  const int64_t cap[3] = {moe::ceil_div(M, kBigM) + max_slots,
                          static_cast<int64_t>(max_slots) * moe::ceil_div(std::max<int64_t>(M, 1), kSmallM),
                          moe::ceil_div(M, kSmallM) + max_slots};
  size_t at = 0;
  auto take = [&](size_t n) { size_t p = at; at = moe::align_up(at + n, 256); return p; };
  w.h = take(static_cast<size_t>(M) * I * moe::elem_bytes(dt));
  for (int t = 0; t < 3; ++t) {
    w.cap[t] = static_cast<int>(std::min<int64_t>(cap[t], 0x3fffffff));
    w.tab_slot[t] = take(sizeof(int32_t) * w.cap[t]);
    w.tab_row0[t] = take(sizeof(int32_t) * w.cap[t]);
    w.tab_rend[t] = take(sizeof(int32_t) * w.cap[t]);
  }
  w.n_tiles = take(3 * sizeof(int32_t));
  w.split_cap = static_cast<int>(std::min<int64_t>(static_cast<int64_t>(max_slots) * kRemTiles + kConvCap, 0x3fffffff));
  w.split_slot = take(2 * sizeof(int32_t) * w.split_cap);
  w.split_row0 = take(2 * sizeof(int32_t) * w.split_cap);
  w.split_rend = take(2 * sizeof(int32_t) * w.split_cap);
  w.split_counts = take(8 * sizeof(int32_t));
  w.mid_slot = take(sizeof(int32_t) * max_slots);  // at most one 128-row tile per range
  w.mid_row0 = take(sizeof(int32_t) * max_slots);
  w.mid_rend = take(sizeof(int32_t) * max_slots);
  w.alt_slot = take(sizeof(int32_t) * w.cap[kG256]);  // the gate/up GEMM's 256-row table without 128-row tails
  w.alt_row0 = take(sizeof(int32_t) * w.cap[kG256]);
  w.alt_rend = take(sizeof(int32_t) * w.cap[kG256]);
  w.steal = take(9 * kStealStride * sizeof(int32_t));  // the gate/up launch's per-XCD counters
  w.bytes = at;
  return w;
}

// Caller-owned events recorded around the two GEMM launches (profiling only;
// null when not profiling).
hipError_t mark(hipEvent_t const* ev, int i, hipStream_t s) {
  return ev ? hipEventRecord(ev[i], s) : hipSuccess;
}

// A 256-row tiling runs with its 128-row and 64-row companion tables in one
// mixed launch (wnt: bf16 weights loaded non-temporally); the 64-row tilings
// run alone.
template <bool kBf16, int EPI, int NMAT>
void launch_gemm(bool small, bool wnt, const GemmArgs& p, const GemmArgs& mid, const GemmArgs& companion,
                 unsigned grid, hipStream_t s) {
  if (small) gemm_kernel<kBf16, NMAT, EPI, kSmallM, 1><<<grid, 256, 0, s>>>(p);
  else if constexpr (kBf16) {
    if (wnt) gemm_mixed_kernel<kBf16, NMAT, EPI, true><<<grid, 256, 0, s>>>(p, mid, companion);
    else gemm_mixed_kernel<kBf16, NMAT, EPI><<<grid, 256, 0, s>>>(p, mid, companion);
  } else {
    gemm_mixed_kernel<kBf16, NMAT, EPI><<<grid, 256, 0, s>>>(p, mid, companion);
  }
}

// Phase 1 (gate/up or W1) and phase 2 (down or W2), each on its own tile table.
template <bool kBf16>
int launch_ffn(const GemmArgs& p1, bool small1, unsigned grid1, const GemmArgs& m1, const GemmArgs& t1,
               const GemmArgs& p2, bool small2, unsigned grid2, const GemmArgs& m2, const GemmArgs& t2, bool swiglu,
               bool wnt1, bool wnt2, hipEvent_t const* ev, hipStream_t s) {
  if (int rc = moe::hip_status(mark(ev, 0, s), "moe_expert_ffn timing event")) return rc;
  if (swiglu) launch_gemm<kBf16, kEpiSwiGLU, 2>(small1, wnt1, p1, m1, t1, grid1, s);
  else launch_gemm<kBf16, kEpiGELU, 1>(small1, wnt1, p1, m1, t1, grid1, s);
  if (int rc = moe::hip_status(hipGetLastError(), "moe_expert_ffn gate/up launch")) return rc;
  if (int rc = moe::hip_status(mark(ev, 1, s), "moe_expert_ffn timing event")) return rc;
  launch_gemm<kBf16, kEpiStore, 1>(small2, wnt2, p2, m2, t2, grid2, s);
  if (int rc = moe::hip_status(hipGetLastError(), "moe_expert_ffn down launch")) return rc;
  return moe::hip_status(mark(ev, 2, s), "moe_expert_ffn timing event");
}

// AUTO rule, per GEMM, from the slot sizes.  Cost model in "row-tile units":
// a 256-row tile costs 1, a 64-row tile kSmallCost (a quarter of the work at a
// lower MFMA efficiency); a grid is charged at least one full wave of the 256
// CUs.  The 256-row tiling counts its short-range tiles (64-row) at kSmallCost.
// The cheapest tiling wins; ties keep the 256-row tiles.  kSmallCost is fitted
// to the measured crossover table (DeepSeek-V2-, Mixtral- and DBRX-shaped
// routing and EPS-MoE's single-expert shapes).
constexpr int kComputeUnits = 256;
Kind pick_kind(int64_t g256, int64_t g256_rem, int64_t d64, int64_t g64, int col_tiles) {
  auto cost = [&](double tiles) {
    return std::max(tiles * col_tiles, static_cast<double>(kComputeUnits));
  };
  // g256_rem: the 256-row tiling's 64- and 128-row tiles (both at kSmallCost)
  const double c256 = cost(static_cast<double>(g256) + kSmallCost * static_cast<double>(g256_rem));
  const double cd64 = kSmallCost * cost(static_cast<double>(d64)), cg64 = kSmallCost * cost(static_cast<double>(g64));
  if (cg64 < c256 && cg64 <= cd64) return kG64;
  if (cd64 < c256) return kD64;
  return kG256;
}

int ffn_impl(const void* x_perm, const int32_t* row_src, int64_t n_src, moe_dtype dt, int64_t M, int H, int I, int E,
             const int32_t* slot_off, const int32_t* slot_expert, const int32_t* n_slots, int max_slots,
             const void* w_gate, const void* w_up, const void* w_down, moe_act act, moe_gemm_path path, void* y_perm,
             void* workspace, size_t workspace_bytes, int32_t* check, hipEvent_t const* ev, void* stream);

}  // namespace

extern "C" size_t moe_expert_ffn_workspace_bytes(moe_dtype dt, int64_t M, int H, int I, int max_slots) {
  (void)H;
  if (M < 0 || I < 1 || max_slots < 1 || (dt != MOE_F32 && dt != MOE_BF16)) return 0;
  return ws_layout(dt, M, I, max_slots).bytes;
}

extern "C" int moe_expert_ffn(const void* x_perm, const int32_t* row_src, int64_t n_src, moe_dtype dt, int64_t M,
                              int H, int I, int E, const int32_t* slot_off, const int32_t* slot_expert,
                              const int32_t* n_slots, int max_slots, const void* w_gate, const void* w_up,
                              const void* w_down, moe_act act, moe_gemm_path path, void* y_perm, void* workspace,
                              size_t workspace_bytes, int32_t* check, void* stream) {
  return ffn_impl(x_perm, row_src, n_src, dt, M, H, I, E, slot_off, slot_expert, n_slots, max_slots, w_gate, w_up,
                  w_down, act, path, y_perm, workspace, workspace_bytes, check, nullptr, stream);
}

extern "C" int moe_expert_ffn_profiled(const void* x_perm, const int32_t* row_src, int64_t n_src, moe_dtype dt,
                                       int64_t M, int H, int I, int E, const int32_t* slot_off,
                                       const int32_t* slot_expert, const int32_t* n_slots, int max_slots,
                                       const void* w_gate, const void* w_up, const void* w_down, moe_act act,
                                       moe_gemm_path path, void* y_perm, void* workspace, size_t workspace_bytes,
                                       int32_t* check, void* const* events, void* stream) {
  if (!events || !events[0] || !events[1] || !events[2])
    return moe::fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn_profiled: needs three events");
  const hipEvent_t ev[3] = {static_cast<hipEvent_t>(events[0]), static_cast<hipEvent_t>(events[1]),
                            static_cast<hipEvent_t>(events[2])};
  return ffn_impl(x_perm, row_src, n_src, dt, M, H, I, E, slot_off, slot_expert, n_slots, max_slots, w_gate, w_up,
                  w_down, act, path, y_perm, workspace, workspace_bytes, check, ev, stream);
}

namespace {

int ffn_impl(const void* x_perm, const int32_t* row_src, int64_t n_src, moe_dtype dt, int64_t M, int H, int I, int E,
             const int32_t* slot_off, const int32_t* slot_expert, const int32_t* n_slots, int max_slots,
             const void* w_gate, const void* w_up, const void* w_down, moe_act act, moe_gemm_path path, void* y_perm,
             void* workspace, size_t workspace_bytes, int32_t* check, hipEvent_t const* ev, void* stream) {
  using namespace moe;
  if (dt != MOE_F32 && dt != MOE_BF16) return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn: unknown dtype %d", (int)dt);
  if (act != MOE_SWIGLU && act != MOE_GELU) return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn: unknown activation");
  if (path != MOE_GEMM_AUTO && path != MOE_GEMM_GROUPED && path != MOE_GEMM_DENSE && path != MOE_GEMM_GROUPED_SMALL)
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
  if (row_src && (n_src < 0 || n_src * H * elem_bytes(dt) >= kGatherLimit))
    return fail(n_src < 0 ? MOE_ERR_INVALID_ARG : MOE_ERR_UNSUPPORTED,
                "moe_expert_ffn: a gathered input of n_src=%lld rows must stay below %lld bytes", (long long)n_src,
                (long long)kGatherLimit);
  for (const void* p : {x_perm, w_gate, w_up, w_down, static_cast<const void*>(y_perm), static_cast<const void*>(workspace)})
    if (p && !aligned16(p)) return fail(MOE_ERR_INVALID_ARG, "moe_expert_ffn: operands must be 16-byte aligned");
  const WsLayout w = ws_layout(dt, M, I, max_slots);
  if (workspace_bytes < w.bytes)
    return fail(MOE_ERR_WORKSPACE, "moe_expert_ffn: workspace has %zu bytes, needs %zu", workspace_bytes, w.bytes);
  if (M == 0) return MOE_OK;

  const hipStream_t s = as_stream(stream);
  const int nt1 = static_cast<int>(ceil_div(I, act == MOE_SWIGLU ? kTileN / 2 : kTileN));
  // The gate/up GEMM runs a range's last tile of at most 128 rows as a 128-row
  // tile when it is bf16 SwiGLU (a register epilogue): half the MFMA work of a
  // 256-row tile for the same weight reads (measured faster on the Mixtral
  // shape and on DeepSeek-V2's 12 column tiles at T = 4096).  The down GEMM
  // keeps the 256-row tiles: there the extra blocks land in an already short
  // last round (measured slower on the Mixtral shape).
  const bool gateup_mid = dt == MOE_BF16 && act == MOE_SWIGLU;
  const int mid_cap_rows = gateup_mid ? 128 : 0;
  const int nt2 = static_cast<int>(ceil_div(H, kTileN));
  // GROUPED: 256-row tiles covering each slot.  GROUPED_SMALL: 64-row tiles
  // covering each slot.  DENSE: the padded batch in 64-row tiles.  AUTO: per
  // GEMM, from the slot sizes read back here.
  Kind k1 = path == MOE_GEMM_DENSE ? kD64 : path == MOE_GEMM_GROUPED_SMALL ? kG64 : kG256, k2 = k1;
  int m_pad = 0;
  int64_t exact[3] = {-1, -1, -1};  // tiles per kind, when known on the host
  int64_t exact_rem = -1;             // the 256-row tiling's 64-row short-range and 128-row tiles
  if (path == MOE_GEMM_DENSE || path == MOE_GEMM_AUTO) {
    // slot sizes, with consecutive slots of one expert merged into one range
    // exactly as the tile tables merge them
    std::vector<int32_t> off(static_cast<size_t>(max_slots) + 2), se(static_cast<size_t>(max_slots));
    if (int rc = hip_status(hipMemcpyAsync(off.data(), slot_off, sizeof(int32_t) * (max_slots + 1),
                                           hipMemcpyDeviceToHost, s), "moe_expert_ffn slot readback")) return rc;
    if (int rc = hip_status(hipMemcpyAsync(&off[max_slots + 1], n_slots, sizeof(int32_t), hipMemcpyDeviceToHost, s),
                            "moe_expert_ffn slot readback")) return rc;
    if (int rc = hip_status(hipMemcpyAsync(se.data(), slot_expert, sizeof(int32_t) * max_slots,
                                           hipMemcpyDeviceToHost, s), "moe_expert_ffn slot readback")) return rc;
    if (int rc = hip_status(hipStreamSynchronize(s), "moe_expert_ffn slot readback")) return rc;
    const int n = std::min(std::max(off[max_slots + 1], 0), max_slots);
    int64_t largest = 0, active = 0, g256 = 0, g256_rem = 0, g256_mid = 0, g64 = 0;
    for (int i = 0; i < n;) {
      int last = i + 1;
      while (last < n && se[last] == se[i]) ++last;
      const int64_t r = std::max<int64_t>(0, std::min<int64_t>(std::max(off[last], 0), M) -
                                                 std::min<int64_t>(std::max(off[i], 0), M));
      largest = std::max(largest, r);
      if (r > 0) ++active;
      // the 256-row tiling: a range of at most kRemTiles x 64 rows as 64-row
      // tiles, else 256-row tiles; for the gate/up GEMM the last as a 128-row
      // tile when it holds at most 128 rows (the tile tables' rule)
      const bool short_range = r > 0 && r <= static_cast<int64_t>(kRemTiles) * kSmallM;
      g256 += short_range ? 0 : ceil_div(r, kBigM);
      g256_rem += short_range ? ceil_div(r, kSmallM) : 0;
      g256_mid += !short_range && mid_cap_rows > 0 && r % kBigM > 0 && r % kBigM <= mid_cap_rows;
      g64 += ceil_div(r, kSmallM);
      i = last;
    }
    m_pad = static_cast<int>(ceil_div(std::max<int64_t>(largest, 1), kSmallM) * kSmallM);
    exact[kG256] = g256;
    exact_rem = g256_rem;
    exact[kD64] = active * (m_pad / kSmallM);
    exact[kG64] = g64;
    if (path == MOE_GEMM_AUTO) {
      k1 = pick_kind(g256 - g256_mid, g256_rem + g256_mid, exact[kD64], g64, nt1);
      k2 = pick_kind(g256, g256_rem, exact[kD64], g64, nt2);
    }
  }
  if ((k1 == kD64 || k2 == kD64) && exact[kD64] > w.cap[kD64])
    return fail(MOE_ERR_WORKSPACE, "moe_expert_ffn: dense path needs %lld tiles", (long long)exact[kD64]);

  // Grids: exact tile counts when read back, else bounds; blocks past the
  // tables exit at once.  A 256-row tiling's tables hold at most
  // floor(M / 256) + (ranges x max(1, kRemTiles)) tiles, ranges <= max_slots
  // (a range's 128-row tile takes the place of its last 256-row tile), plus 3
  // more per re-listed trailing row tile (at most ceil(256 / nt) of those),
  // plus the rounding of the 256- and 128-row parts to 8 blocks each; a mixed
  // launch that deals its tail at run time needs kStealExtra more blocks per
  // XCD and a block per XCD for each of the three tables' uneven shares.
  auto grid = [&](Kind t, int nt) {
    int64_t blocks;
    if (t == kG256) {
      const int64_t both = exact[kG256] >= 0 ? exact[kG256] + exact_rem
                                             : M / kBigM + static_cast<int64_t>(max_slots) * std::max(1, kRemTiles);
      blocks = both * nt + 3 * ceil_div(kWaveBlocks, nt) * nt + 16;
      if (blocks >= kStealMinTiles) blocks += 8 * (kStealExtra + 4);  // else the launch keeps the fixed schedule
    } else {
      blocks = (exact[t] >= 0 ? exact[t] : static_cast<int64_t>(w.cap[t])) * nt;
    }
    return std::max<int64_t>(1, blocks);
  };
  // block and tile indices are 32-bit in the kernels
  const int64_t blocks1 = grid(k1, nt1), blocks2 = grid(k2, nt2);
  if (std::max(blocks1, blocks2) >= (int64_t(1) << 31) - kWaveBlocks)
    return fail(MOE_ERR_UNSUPPORTED, "moe_expert_ffn: %lld blocks exceed 32-bit grid indexing",
                static_cast<long long>(std::max(blocks1, blocks2)));
  const unsigned grid1 = static_cast<unsigned>(blocks1), grid2 = static_cast<unsigned>(blocks2);

  char* ws = static_cast<char*>(workspace);
  int32_t* n_tiles = reinterpret_cast<int32_t*>(ws + w.n_tiles);
  auto tab_slot = [&](int t) { return reinterpret_cast<int32_t*>(ws + w.tab_slot[t]); };
  auto tab_row0 = [&](int t) { return reinterpret_cast<int32_t*>(ws + w.tab_row0[t]); };
  auto tab_rend = [&](int t) { return reinterpret_cast<int32_t*>(ws + w.tab_rend[t]); };
  // 256-row tables come with a 64-row companion table per GEMM that runs on
  // them: ranges of <= 64 rows, and trailing row tiles re-listed when that
  // shortens the launch's last round
  int32_t* split_counts = reinterpret_cast<int32_t*>(ws + w.split_counts);
  TileSplit split{};
  split.nt[0] = k1 == kG256 ? nt1 : 0;
  split.nt[1] = k2 == kG256 ? nt2 : 0;
  split.cap = w.split_cap;
  split.rem_tiles = kRemTiles;
  split.small_cost = static_cast<float>(kSmallCost);
  split.slot = reinterpret_cast<int32_t*>(ws + w.split_slot);
  split.row0 = reinterpret_cast<int32_t*>(ws + w.split_row0);
  split.rend = reinterpret_cast<int32_t*>(ws + w.split_rend);
  split.counts = split_counts;
  const bool mid1 = gateup_mid && k1 == kG256;
  split.mid_rows = mid1 ? 128 : 0;
  split.mid_slot = reinterpret_cast<int32_t*>(ws + w.mid_slot);
  split.mid_row0 = reinterpret_cast<int32_t*>(ws + w.mid_row0);
  split.mid_rend = reinterpret_cast<int32_t*>(ws + w.mid_rend);
  split.alt_slot = reinterpret_cast<int32_t*>(ws + w.alt_slot);
  split.alt_row0 = reinterpret_cast<int32_t*>(ws + w.alt_row0);
  split.alt_rend = reinterpret_cast<int32_t*>(ws + w.alt_rend);
  int32_t* const steal = reinterpret_cast<int32_t*>(ws + w.steal);
  split.steal = steal;
  auto build = [&](Kind t) {
    const int mode = t == kD64 ? kPadded : kCover;
    const int bm = t == kG256 ? kBigM : kSmallM;
    tiles_kernel<<<1, 256, 0, s>>>(slot_off, slot_expert, n_slots, max_slots, M, E, mode, bm, m_pad, 1, w.cap[t],
                                   tab_slot(t), tab_row0(t), tab_rend(t), n_tiles + t,
                                   t == kG256 ? split : TileSplit{}, check);
    return hip_status(hipGetLastError(), "moe_expert_ffn tile-table launch");
  };
  if (int rc = build(k1)) return rc;
  if (k2 != k1)
    if (int rc = build(k2)) return rc;

  GemmArgs p1{};
  p1.A = x_perm;
  p1.a_rows = row_src;  // the gate/up GEMM gathers its rows when given a row map
  p1.a_n = n_src;
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
  p2.a_rows = nullptr;
  p2.B0 = w_down;
  p2.B1 = nullptr;
  p2.C = y_perm;
  p2.K = I;
  p2.N = H;
  p2.n_col_tiles = nt2;
  // The gate/up launch deals its tail at run time (its 256- and 128-row tiles
  // are short enough to even out the XCDs' clocks: 1.4-3.5% faster on the
  // Mixtral shape in same-box A/Bs); the down GEMM keeps the fixed schedule
  // (its tiles last longer than the XCDs drift apart, and the counters cost
  // it 0.6%).
  p1.steal = k1 == kG256 ? steal : nullptr;
  auto on = [&](GemmArgs& g, Kind t, int which) {
    g.tile_slot = tab_slot(t);
    g.tile_row0 = tab_row0(t);
    g.tile_rend = tab_rend(t);
    g.n_tiles = t == kG256 ? split_counts + 2 * which : n_tiles + t;
  };
  on(p1, k1, 0);
  on(p2, k2, 1);
  if (mid1) {  // the gate/up GEMM's 256-row table without its 128-row tails
    p1.tile_slot = split.alt_slot;
    p1.tile_row0 = split.alt_row0;
    p1.tile_rend = split.alt_rend;
  }
  // the 64-row companion tables of the mixed launches
  auto companion = [&](const GemmArgs& g, int which) {
    GemmArgs q = g;
    q.tile_slot = split.slot + static_cast<int64_t>(which) * w.split_cap;
    q.tile_row0 = split.row0 + static_cast<int64_t>(which) * w.split_cap;
    q.tile_rend = split.rend + static_cast<int64_t>(which) * w.split_cap;
    q.n_tiles = split_counts + 2 * which + 1;
    return q;
  };
  const GemmArgs t1 = companion(p1, 0), t2 = companion(p2, 1);
  // the 128-row table of the gate/up GEMM (count split_counts[4]; empty when
  // not used); the down GEMM's is always empty (split_counts[5] = 0)
  auto mid_table = [&](const GemmArgs& g, int which) {
    GemmArgs q = g;
    q.tile_slot = split.mid_slot;
    q.tile_row0 = split.mid_row0;
    q.tile_rend = split.mid_rend;
    q.n_tiles = split_counts + 4 + which;
    return q;
  };
  const GemmArgs m1 = mid_table(p1, 0), m2 = mid_table(p2, 1);
  const bool swiglu = act == MOE_SWIGLU;
  // Weight rows go through the caches with the non-temporal hint when few row
  // tiles share an expert's weights (M / E rows per expert on average) and the
  // launch is large enough to contend for the caches (up to one round of 256
  // tiles, counting a partial row tile per expert): they then give way to the
  // activation rows, which every column tile of a row tile reads again.  Timed
  // against plain loads on the DeepSeek-V2-, Mixtral- and DBRX-shaped
  // routings: the hint pays on the gate/up GEMM up to 1024 rows per expert
  // (four row tiles; its activation rows serve 2I / 256 column tiles) and on
  // the down GEMM below 256 (H / 256 column tiles), and costs time above; on a
  // single expert of 512 rows with 12 column tiles (24 tiles) it cost 40%.
  const int64_t per_expert = M / std::max(E, 1);
  const int64_t row_tiles = ceil_div(M, kBigM) + E;
  const bool big_launch1 = row_tiles * nt1 >= kComputeUnits, big_launch2 = row_tiles * nt2 >= kComputeUnits;
  const bool wnt1 = per_expert <= 1024 && big_launch1, wnt2 = per_expert < 256 && big_launch2;
  return dt == MOE_BF16
             ? launch_ffn<true>(p1, k1 != kG256, grid1, m1, t1, p2, k2 != kG256, grid2, m2, t2, swiglu, wnt1, wnt2,
                                ev, s)
             : launch_ffn<false>(p1, k1 != kG256, grid1, m1, t1, p2, k2 != kG256, grid2, m2, t2, swiglu, false, false,
                                 ev, s);
}

}  // namespace
