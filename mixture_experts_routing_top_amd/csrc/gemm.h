// The tiled MFMA GEMM shared by the forward FFN and its backward pass.
//
// Source: EPS-MoE review, section 3 (the gate, up and down GEMMs are the
// compute-bound part of an MoE layer; GroupGemm runs every expert's product in
// one kernel; DenseGemm runs a padded uniform batch).  The backward pass adds
// the transposed products of the same layer (PopFetcher wiki, method: the
// backward pass of MoE training).
//
// gfx950 mapping.  A block is 256 threads (4 waves, one per SIMD) computing a
// BM x 256 output tile; with BM = 256 each wave owns 128 x 128 as 4 x 4 MFMA
// tiles of 32 x 32 (v_mfma_f32_32x32x16_bf16, or v_mfma_f32_32x32x2f32 for
// fp32), 256 accumulator registers.  K advances 128 bytes per row per step (64
// bf16 / 32 fp32).  bf16 256-row tiles fetch their operands straight into LDS
// (buffer_load ... lds: no register staging, no LDS write instructions), into
// two A stages and three weight stages of swizzled 128-byte rows; the other
// tiles stage the next step through registers into two LDS stages of padded
// rows (144-byte pitch).  Both read conflict-free 16-byte fragments, take one
// barrier per step and pin the instruction order.  Operands are read with raw
// buffer loads whose range ends at the last valid row, so rows past the end
// read as zero and need no clamping.  Blocks are remapped so each of the 8 XCDs
// works on a contiguous run of tiles, ordered 8 row tiles by N columns, which
// keeps the A and B tiles that neighbouring blocks share inside that XCD's L2.
// The weight fragment is the MFMA's first operand, so the accumulators come out
// transposed: each lane holds four adjacent output columns of one row, which
// the epilogue writes with one 8-byte (bf16) or 16-byte (fp32) store.  One
// launch can run three tile heights (gemm_mixed_kernel): 256-row tiles, then
// 128- and 64-row tiles in the grid's last blocks, over one shared LDS array.
// bf16 256-row tiles can also read an operand K-major ([K, N] with N
// contiguous: the backward's weights and its weight gradients' activations):
// its stages then hold 64 rows of one K index each, and the MFMA fragments
// come from gfx950's transposed LDS read (ds_read_b64_tr_b16).
// Each output row depends only on its own input row and the fixed K order, so
// a row's value does not depend on the tile, slot or path that computes it.
#pragma once

#include <type_traits>

#include "common.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Epilogues.  Forward: SwiGLU / GELU activation to the dtype, or a plain store.
// Backward: an fp32 store (d_h), and the recomputed gate/up (or W1)
// pre-activations met with d_h (read from aux, fp32 [M, I]): the activation
// gradient ([M, 2I] d_g then d_u, or [M, I] d_z, into C) and h ([M, I], into
// C2), rounded to the dtype.
enum Epi {
  kEpiSwiGLU = 0, kEpiGELU = 1, kEpiStore = 2, kEpiStoreF32 = 3, kEpiSwiGLUGrad = 4, kEpiGELUGrad = 5
};

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
constexpr int kStagedStoreMinBM = 128;  // bf16 tiles this tall stage their SwiGLU or plain stores in LDS

struct GemmArgs {
  const void* A;   // [M, K]; weight-gradient mode: [Mw, ld] (rows of transposed activations)
  const void* B0;  // [E, N, K]; weight-gradient mode: [N, ld]
  const void* B1;  // [E, N, K] or null
  void* C;         // [M, N] (the epilogue says how it is laid out)
  int64_t M;
  int K, N, E;
  const int32_t* slot_off;
  const int32_t* slot_expert;
  const int32_t* tile_slot;
  const int32_t* tile_row0;
  const int32_t* tile_rend;  // end row of the range the tile belongs to
  const int32_t* n_tiles;
  int n_col_tiles;
  // backward only
  const float* aux;    // pre-activations read by the backward epilogues
  int ld;              // weight-gradient mode: row length of A and B (elements)
  const int32_t* seg;  // weight-gradient mode: expert e's K range is [seg[e], seg[e+1])
  int Mw;              // weight-gradient mode: rows of A (output rows per expert)
  int c_split;         // weight-gradient mode: output rows >= c_split go to C2
  void* C2;
  // K-major operands (bf16 256-row tiles, template argument KM): A stored as
  // [K rows, lda] (weight-gradient mode: the activations [M, lda], expert e's
  // rows slot_off[e] .. slot_off[e+1] being its K range), the weights as
  // [E, Kb, ldb] (weight-gradient mode: activations [M, ldb] like A).  With
  // k_split > 0 the weights' K range is split: k < k_split reads B0 [E,
  // k_split, ldb], k >= k_split reads B1 (its row k - k_split).
  int lda, ldb, k_split;
  // Gathered A rows (not in weight-gradient or K-major mode): with a_rows set,
  // row r of the M rows is row a_rows[r] of A = [a_n, K]; rows mapped outside
  // [0, a_n) read as zero.  The caller keeps a_n * K * sizeof(T) below
  // kGatherLimit so every offset stays in 31 bits.
  const int32_t* a_rows;
  int64_t a_n;
  // Mixed launches only: eight per-XCD counters and an all-empty word
  // (kStealStride apart, zero at launch) that deal the last tiles of each
  // XCD's share at run time; null: every block's tile follows from its index
  // alone.
  int32_t* steal;
};
constexpr int64_t kGatherLimit = int64_t(0x7e000000);  // bytes of a gathered A
constexpr int kGatherOut = 0x7f000000;                 // an A offset out of range: reads zero

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : static_cast<int>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), n, 0x00020000);
}

__device__ __forceinline__ uint4 bload(__amdgpu_buffer_rsrc_t r, int off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Buffer descriptor in four SGPRs for the LDS-DMA loads below: offsets at or
// past `bytes` read as zero without touching memory.
__device__ __forceinline__ u32x4 dma_rsrc(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const unsigned n = bytes > 0x7fffffff ? 0x7fffffffu : static_cast<unsigned>(bytes);
  u32x4 d;
  d.x = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a));
  d.y = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a >> 32) & 0xffffu);
  d.z = __builtin_amdgcn_readfirstlane(n);
  d.w = 0x00020000u;
  return d;
}

// 16 bytes per lane from global memory straight into LDS: lane i writes
// lds_block + 16 i.  The instruction has no register result; its completion
// is counted by vmcnt and awaited explicitly (wait_vm) before the barrier that
// publishes the stage.
// M0 is set here and nowhere else in these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void load_lds(const u32x4& r, int off, unsigned lds_block) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_block), "v"(off), "s"(r)
               : "m0");
}
// The same with the non-temporal hint: the lines are the first the caches
// give up, for data that no other tile will read again soon.
__device__ __forceinline__ void load_lds_nt(const u32x4& r, int off, unsigned lds_block) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :
               : "s"(lds_block), "v"(off), "s"(r)
               : "m0");
}
template <bool NT>
__device__ __forceinline__ void load_lds_hint(const u32x4& r, int off, unsigned lds_block) {
  if constexpr (NT) load_lds_nt(r, off, lds_block);
  else load_lds(r, off, lds_block);
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(n) with the other counters left alone (n < 64).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0xF70);
}

// Direct-to-LDS stage rows hold 128 bytes (one K step) as eight 16-byte chunks,
// chunk c stored at c ^ swz(row): any 16 consecutive rows read at one logical
// chunk hit 16 distinct 16-byte bank groups.  swz depends on row % 32 only.
__device__ __forceinline__ int swz(int row) { return (row ^ ((row >> 3) & 3)) & 7; }

// K-major stage rows hold 512 bytes (256 elements of one K index) as 32
// chunks of 16 bytes; logical chunk c is stored at c ^ kswz(row), which moves
// whole 32-byte pairs of chunks: by 0, 5, 2, 7 pairs for row % 4 = 0..3.  A
// transposed fragment read takes 32 bytes from each of four rows r..r+3 (r a
// multiple of 4) per 16 lanes, and 64 bytes from each per 32 lanes; these
// shifts put the four (or eight) pieces in distinct 32-byte bank groups.
__device__ __forceinline__ int kswz(int row) { return (((row & 2) | ((row & 1) * 5)) << 1); }

// Four adjacent outputs: fp32 as one 16-byte store, bf16 rounded to nearest
// even (v_cvt_pk_bf16_f32) as one 8-byte store.
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void store4(float* p, const float v[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
// The forward activations, shared with the backward pass that rebuilds h from
// the fp32 pre-activations, so both round the same value.  SwiGLU: silu(g) u
// with g / (1 + 2^(-g log2 e)) on the hardware exp2 and reciprocal (an
// infinite exponent gives 0); GELU: the exact erf form.
__device__ __forceinline__ float swiglu_h(float g, float u) {
  return g * __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(g * -1.4426950408889634f)) * u;
}
__device__ __forceinline__ float gelu_h(float z) { return 0.5f * z * (1.f + erff(z * 0.70710678118654752f)); }

__device__ __forceinline__ void store4(uint16_t* p, const float v[4]) {
  const bf16x2 lo = __builtin_convertvector((f32x2{v[0], v[1]}), bf16x2);
  const bf16x2 hi = __builtin_convertvector((f32x2{v[2], v[3]}), bf16x2);
  *reinterpret_cast<uint2*>(p) = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// BM rows x 256 weight rows per block; the 4 waves form a WM x (4/WM) grid.
// BM = 256, WM = 2: each wave owns 128 x 128 (4 x 4 MFMA tiles).
// BM = 64,  WM = 1: each wave owns  64 x 64  (2 x 2 MFMA tiles).
// kWgrad: weight-gradient mode.  Tiles are (expert, 256 output rows, 256
// output columns); the reduction runs over expert e's rows, which the caller
// has transposed into the K range [seg[e], seg[e+1]) (a multiple of the K step,
// zero-padded) of A [Mw, ld] and B [N, ld]; output rows below c_split go to
// C [E, c_split, N], the others to C2 [E, Mw - c_split, N].
// LDS bytes one block of a tiling needs (operand stages, or the epilogue's
// staging tile where that is larger).
template <bool kBf16, int NMAT, int EPI, int BM, int WM, bool kWgrad>
constexpr int gemm_lds_bytes() {
  constexpr bool kDTL = kBf16 && (BM == 256 || BM == 128);
  constexpr bool kDTL64 = kBf16 && BM == 64 && !kWgrad;
  constexpr int kStageBytes = (BM + kTileN) * kRowBytes;
  constexpr int kStagedEpi = (!kWgrad && (EPI == kEpiGELU || EPI == kEpiSwiGLUGrad || EPI == kEpiGELUGrad ||
                                          EPI == kEpiStoreF32))
                                 ? (BM / WM) * (kTileN + 4) * 4 : 0;
  constexpr int kDtlBytes = kDTL ? 2 * BM * 128 + 3 * kTileN * 128 : 4 * (BM + kTileN) * 128;
  return (kDTL || kDTL64) ? (kDtlBytes > kStagedEpi ? kDtlBytes : kStagedEpi) : 2 * kStageBytes;
}

// The GEMM kernels' LDS: one array that every tiling of a launch shares.
constexpr int kGemmLdsBytes = 160 * 1024;
__shared__ __align__(1024) char gemm_lds[kGemmLdsBytes];

// One block's tile: `b` is its index in the grid of this tiling (b & 7 its
// XCD); it uses the first gemm_lds_bytes of gemm_lds.
// WNT: the bf16 weight rows are loaded with the non-temporal hint.
template <bool kBf16, int NMAT, int EPI, int BM, int WM, bool kWgrad = false, int KM = 0, bool WNT = false>
__device__ __forceinline__ void gemm_tile(const GemmArgs g, const int b) {
  char* const lds = gemm_lds;
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
  // K-major operands: bit 0 A (weight-gradient mode only), bit 1 the weights
  constexpr bool kAK = (KM & 1) != 0, kBK = (KM & 2) != 0;
  static_assert(KM == 0 || (kBf16 && BM == 256 && WM == 2 && NMAT == 1 && (!kAK || kWgrad)),
                "K-major operands: bf16 256-row tiles of one weight matrix; K-major A in weight-gradient mode");
  // bf16 tiles load their operands straight into LDS (unpadded rows): 256- and
  // 128-row tiles (weight gradients included) in two A stages and three weight
  // stages, 64-row tiles in four stages of both; fp32 tiles stage them through
  // registers into two padded stages
  constexpr bool kDTL = kBf16 && (BM == 256 || BM == 128);
  constexpr bool kDTL64 = kBf16 && BM == 64 && !kWgrad;
  constexpr int kLdsBytes = gemm_lds_bytes<kBf16, NMAT, EPI, BM, WM, kWgrad>();

  // ---- which tile: XCD-contiguous runs, grouped raster inside a run --------
  const int NT = g.n_col_tiles;
  const int MTw = kWgrad ? (g.Mw + BM - 1) / BM : 0;       // row tiles per expert (weight gradients)
  const int total_m = kWgrad ? g.E * MTw : *g.n_tiles;
  // weight gradients: 8 equal shares of each expert's tiles (grid rounded up to them)
  const int total = kWgrad ? 8 * g.E * ((MTw * NT + 7) >> 3) : total_m * NT;
  if (b >= total) return;
  int mt, nt;
  if constexpr (kWgrad) {
    // experts differ in K (their row counts): give each XCD an equal, contiguous
    // share of every expert's tiles, so no XCD holds all of a hot expert
    const int per_e = MTw * NT;
    const int xcd = b & 7, pos = b >> 3;
    const int e_ = pos / ((per_e + 7) >> 3);
    const int in_e = pos - e_ * ((per_e + 7) >> 3);
    const int t_ = xcd * ((per_e + 7) >> 3) + in_e;     // tile index inside the expert
    if (e_ >= g.E || t_ >= per_e) return;
    const int gm = t_ / (kGroupM * NT);
    const int gs = min(kGroupM, MTw - gm * kGroupM);
    const int li_ = t_ - gm * kGroupM * NT;
    mt = e_ * MTw + gm * kGroupM + li_ % gs;
    nt = li_ / gs;
  } else {
    const int xcd = b & 7, q = total >> 3, rem = total & 7;
    const int l = xcd * q + min(xcd, rem) + (b >> 3);
    const int grp = l / (kGroupM * NT);
    const int gsz = min(kGroupM, total_m - grp * kGroupM);
    const int li = l - grp * kGroupM * NT;
    mt = grp * kGroupM + li % gsz;
    nt = li / gsz;
  }

  int K, e, m_valid;
  int64_t r0;
  const int N = g.N;
  const int n0 = nt * NSUB;
  const int n_valid = min(NSUB, N - n0);
  const T* A;
  int64_t wofs, row_b;
  if constexpr (kWgrad) {
    e = __builtin_amdgcn_readfirstlane(mt / MTw);
    r0 = __builtin_amdgcn_readfirstlane((mt - e * MTw) * BM);
    m_valid = __builtin_amdgcn_readfirstlane(static_cast<int>(min<int64_t>(BM, g.Mw - r0)));
    if constexpr (KM != 0) {
      // expert e's rows of the activations, read in place: row k0 + k is K index k
      const int64_t lo = min<int64_t>(max(__builtin_amdgcn_readfirstlane(g.slot_off[e]), 0), g.M);
      const int64_t hi = min<int64_t>(max<int64_t>(__builtin_amdgcn_readfirstlane(g.slot_off[e + 1]), lo), g.M);
      K = static_cast<int>(hi - lo);
      row_b = 0;
      A = static_cast<const T*>(g.A) + lo * g.lda + r0;
      wofs = lo * g.ldb + n0;
    } else {
      // uniform across the block: keep the buffer descriptors in scalar registers
      const int k0 = __builtin_amdgcn_readfirstlane(g.seg[e]);
      K = __builtin_amdgcn_readfirstlane(g.seg[e + 1]) - k0;
      row_b = static_cast<int64_t>(g.ld) * S;
      A = static_cast<const T*>(g.A) + r0 * g.ld + k0;
      wofs = static_cast<int64_t>(n0) * g.ld + k0;
    }
  } else {
    const int s = g.tile_slot[mt];
    r0 = g.tile_row0[mt];
    const int64_t rend = min<int64_t>(g.tile_rend[mt], g.M);
    e = g.slot_expert[s];
    if (r0 >= rend || e < 0 || e >= g.E) return;
    K = g.K;
    m_valid = static_cast<int>(min<int64_t>(BM, rend - r0));
    row_b = static_cast<int64_t>(K) * S;  // bytes per operand row
    A = static_cast<const T*>(g.A) + r0 * K;
    if constexpr ((KM & 2) != 0)  // expert e's weights [Kb, ldb] from column n0
      wofs = static_cast<int64_t>(e) * (g.k_split > 0 ? g.k_split : K) * g.ldb + n0;
    else
      wofs = (static_cast<int64_t>(e) * N + n0) * K;
  }

  // gathered A rows: offsets are taken from the row map against A's base
  const bool gat = !kWgrad && KM == 0 && g.a_rows != nullptr;
  if (gat) A = static_cast<const T*>(g.A);
  // byte offset of tile row `row` of a gathered A (out of range past m_valid
  // or for a row mapped outside A)
  auto gather_off = [&](int row) -> int {
    if (row >= m_valid) return kGatherOut;
    const int src = g.a_rows[r0 + row];
    return (src >= 0 && src < g.a_n) ? src * static_cast<int>(row_b) : kGatherOut;
  };
  const __amdgpu_buffer_rsrc_t ra = gat ? rsrc(A, g.a_n * row_b) : rsrc(A, m_valid * row_b);
  const __amdgpu_buffer_rsrc_t rb0 = rsrc(static_cast<const T*>(g.B0) + wofs, n_valid * row_b);
  const __amdgpu_buffer_rsrc_t rb1 =
      NMAT > 1 ? rsrc(static_cast<const T*>(g.B1) + wofs, n_valid * row_b) : rb0;

  // ---- global -> register staging: P x 16 bytes per thread per step -------
  // pass p < PA: A rows 32p..; then 8 passes of weight rows (gate/up: 4 + 4)
  const int tid = threadIdx.x;
  __builtin_assume(tid >= 0 && tid < 256);
  const int lrow = tid >> 3, lchunk = tid & 7;
  const int goff = lrow * static_cast<int>(row_b) + lchunk * 16;  // + pass*32 rows + step*128
  const int pass_b = 32 * static_cast<int>(row_b);
  const int loff = lrow * kRowBytes + lchunk * 16;
  // NST register stages: 64-row tiles keep two steps of loads in flight (one
  // of their K steps is shorter than the load latency); 256-row tiles one
  constexpr int NST = BM == 64 ? 2 : 1;
  uint4 st[NST][P];
  // gathered A: pass p's row offset of this thread (its row lrow + 32 p)
  int aoff[PA];
#pragma unroll
  for (int p = 0; p < PA; ++p) aoff[p] = gat ? gather_off(lrow + 32 * p) + lchunk * 16 : 0;
  auto issue_one = [&](int w, int p, int o, int ao) {
    if (p < PA) st[w][p] = gat ? bload(ra, aoff[p] + ao) : bload(ra, o + p * pass_b);
    else if (NMAT == 1 || p < PA + 4) st[w][p] = bload(rb0, o + (p - PA) * pass_b);
    else st[w][p] = bload(rb1, o + (p - PA - 4) * pass_b);
  };
  // steps past the last one load from an offset out of range: zeros, no memory
  // access (a gathered A reloads step 0's rows instead: no stage past the last
  // step is consumed)
  auto issue = [&](int w, int kt, int nk) {
    const int o = kt < nk ? goff + kt * 128 : 0x7ffff000;
    const int ao = kt < nk ? kt * 128 : 0;
#pragma unroll
    for (int p = 0; p < P; ++p) issue_one(w, p, o, ao);
  };
  auto stash = [&](int stage) {
    char* base = lds + stage * kStageBytes + loff;
#pragma unroll
    for (int p = 0; p < P; ++p) *reinterpret_cast<uint4*>(base + p * 32 * kRowBytes) = st[0][p];
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
      for (int j = 0; j < TN; ++j) acc[i][j] = mma(fb[buf][j], fa[buf][i], acc[i][j]);
  };

  // ---- direct-to-LDS main loop (bf16, 256-row tiles) ------------------------
  // LDS holds two stages of the A rows and three of the 256 weight rows, 128
  // bytes (one K step) per row, swizzled.  Wave w fills the 1 KiB blocks (8
  // rows) 4p + w of a stage, lane i taking row i / 8 and the chunk that lands at
  // i % 8.  A is fetched right after the barrier that frees its stage, the
  // weights a step earlier, and the 16 blocks a wave fetches per step are
  // spread over its four sub-steps.
  auto dtl_main_loop = [&]() {
    constexpr int SA = BM * 128;       // one A stage (two of them)
    constexpr int SBW = kTileN * 128;  // one weight stage (three of them, after the A stages)
    constexpr int PA_ = BM / 32;       // A blocks (8 rows) per wave per step
    constexpr int PB_ = kTileN / 32;   // weight blocks per wave per step
    static_assert(!kDTL || ((PA_ == 8 || PA_ == 4) && PB_ == 8 && NM >= 8),
                  "issue pattern: 8 or 4 A blocks and 8 weight blocks per wave, 3/3/2 weight blocks over the "
                  "first three sub-steps and the A blocks in the fourth, one per odd MFMA");
    const int rb_ = static_cast<int>(row_b);
    const u32x4 da = dma_rsrc(A, (gat ? g.a_n : static_cast<int64_t>(m_valid)) * row_b);
    const u32x4 db0 = dma_rsrc(static_cast<const T*>(g.B0) + wofs, static_cast<int64_t>(n_valid) * row_b);
    const u32x4 db1 = NMAT > 1 ? dma_rsrc(static_cast<const T*>(g.B1) + wofs, static_cast<int64_t>(n_valid) * row_b) : db0;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    // K-major stages hold 64 K rows of 256 elements (512 bytes) each; block
    // 4p + w of a stage is K rows 2(4p + w) and 2(4p + w) + 1, lane i writing
    // 16-byte chunk i % 32 of row i / 32, which holds logical chunk (i % 32) ^
    // kswz(row).  The source row pitch is lda or ldb elements.
    const int ldaB = kAK ? g.lda * S : 0, ldbB = kBK ? g.ldb * S : 0;
    int offA[PA_], offB[PB_];
#pragma unroll
    for (int p = 0; p < PA_; ++p) {
      if constexpr (kAK) {
        const int kr = 2 * (4 * p + wv) + (lane >> 5);
        offA[p] = kr * ldaB + (((lane & 31) ^ kswz(kr)) << 4);
      } else {
        const int row = 8 * (4 * p + wv) + (lane >> 3);
        offA[p] = (gat ? gather_off(row) : row * rb_) + (((lane & 7) ^ swz(row)) << 4);
      }
    }
#pragma unroll
    for (int p = 0; p < PB_; ++p) {
      if constexpr (kBK) {
        const int kr = 2 * (4 * p + wv) + (lane >> 5);
        offB[p] = kr * ldbB + (((lane & 31) ^ kswz(kr)) << 4);
      } else {
        const int row = 8 * (4 * p + wv) + (lane >> 3);
        const int src = (NMAT == 2 && row >= 128) ? row - 128 : row;
        offB[p] = src * rb_ + (((lane & 7) ^ swz(row)) << 4);
      }
    }
    const int nk = KM != 0 ? (K + 63) / 64 : K / 64;
    auto koff = [&](int kt) { return kt < nk ? kt * 128 : 0x7ffff000; };
    // a gathered A's step offset (past the last step: step 0's rows again,
    // never consumed)
    auto koffA = [&](int kt) { return gat ? (kt < nk ? kt * 128 : 0) : koff(kt); };
    // descriptors of step kt for the K-major operands, based at its first K
    // row and ending where the operand's K range ends (an empty range past the
    // last step: its loads read zeros)
    auto kdescA = [&](int kt) -> u32x4 {
      if (!kAK || kt >= nk) return dma_rsrc(A, 0);
      const int64_t o = static_cast<int64_t>(kt) * 64 * g.lda;
      return dma_rsrc(A + o, max<int64_t>(0, (static_cast<int64_t>(K) * g.lda - r0 - o) * S));
    };
    auto kdescB = [&](int kt) -> u32x4 {
      if (!kBK || kt >= nk) return dma_rsrc(g.B0, 0);
      int64_t kr = static_cast<int64_t>(kt) * 64, kend = K;
      const T* base = static_cast<const T*>(g.B0) + wofs;
      if (!kWgrad && g.k_split > 0) {
        if (kr >= g.k_split) {
          base = static_cast<const T*>(g.B1) + wofs;
          kr -= g.k_split;
          kend = K - g.k_split;
        } else {
          kend = g.k_split;
        }
      }
      return dma_rsrc(base + kr * g.ldb, max<int64_t>(0, ((kend - kr) * g.ldb - n0) * S));
    };
    const unsigned lds0 = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(reinterpret_cast<uintptr_t>(lds)));
    // koff: the K offset of a row-major operand's step; dk: a K-major operand's step descriptor
    auto dmaA = [&](int p, int st, int koff, const u32x4& dk) {
      const unsigned dst = lds0 + st * SA + (4 * p + wv) * 1024;
      if constexpr (kAK) load_lds(dk, offA[p], dst);
      else load_lds(da, offA[p] + koff, dst);
    };
    auto dmaB = [&](int p, int st, int koff, const u32x4& dk) {
      const unsigned dst = lds0 + 2 * SA + st * SBW + (4 * p + wv) * 1024;
      if constexpr (kBK) load_lds(dk, offB[p], dst);
      else if (NMAT == 1 || p < PB_ / 2) load_lds_hint<WNT>(db0, offB[p] + koff, dst);
      else load_lds_hint<WNT>(db1, offB[p] + koff, dst);
    };
    constexpr int BS0[4] = {0, 3, 6, 8};  // weight blocks issued in sub-steps 0, 1, 2
    const int sw = swz(lr);
    const int a_rd2 = (wm * (BM / WM) + lr) * 128;
    int b_rd2[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) b_rd2[j] = 2 * SA + (brow(j) + lr) * 128;
    int kofs[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) kofs[kk] = ((2 * kk + lg) ^ sw) << 4;
    // K-major fragments: lane l = 16 q + s (q = l / 16) reads with the
    // transposed 8-byte LDS read ds_read_b64_tr_b16, which hands lane s of a
    // 16-lane group element s % 4 of what lanes 4j + s / 4 (j = 0..3) loaded.
    // So lane s loads K row 8 (q / 2) + s / 4 (+4 for the second read) at
    // columns c0 + 16 (q % 2) + 4 (s % 4) .. + 3, and ends up holding column
    // c0 + l % 32 at K 8 (l / 32) + 0..7: the MFMA operand layout.  kswz
    // depends on the K row mod 4 = s / 4 only, so the per-lane address of a
    // 32-column block is fixed; sub-step kk and the half add immediates.
    int akm_rd[TM], bkm_rd[TN];
    {
      const int q = lane >> 4, s4 = lane & 15;
      const int kb = (8 * (q >> 1) + (s4 >> 2)) * 512 + 8 * (s4 & 3);
#pragma unroll
      for (int i = 0; i < TM; ++i)
        akm_rd[i] = kb + 32 * ((((wm * (BM / WM) + 32 * i) >> 4) + (q & 1)) ^ (kswz(s4 >> 2) >> 1));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bkm_rd[j] = 2 * SA + kb + 32 * ((((wn * CW + 32 * j) >> 4) + (q & 1)) ^ (kswz(s4 >> 2) >> 1));
    }
    auto kfrag = [&](const char* p) {
      typedef short s16x4 __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) s16x4* lds_s16x4;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(p));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4)(p + 4 * 512));
      const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
      return make_uint4(l2.x, l2.y, h2.x, h2.y);
    };
    // fragment read r of a sub-step in the order the MFMAs consume them:
    // A tile 0, weight tiles 0 .. TN-1, A tiles 1 .. TM-1
    auto frag = [&](int sa, int sbw, int kk, int buf, int r) {
      if (r >= 1 && r <= TN) {
        if constexpr (kBK) fb[buf][r - 1] = kfrag(lds + sbw * SBW + bkm_rd[r - 1] + kk * 16 * 512);
        else fb[buf][r - 1] = *reinterpret_cast<const Frag*>(lds + sbw * SBW + b_rd2[r - 1] + kofs[kk]);
      } else {
        const int i = r == 0 ? 0 : r - TN;
        if constexpr (kAK) fa[buf][i] = kfrag(lds + sa * SA + akm_rd[i] + kk * 16 * 512);
        else fa[buf][i] = *reinterpret_cast<const Frag*>(lds + sa * SA + a_rd2 + i * 32 * 128 + kofs[kk]);
      }
    };
    auto mfma1 = [&](int buf, int m) {
      const int i = m / TN, j = m % TN;
      acc[i][j] = mma(fb[buf][j], fa[buf][i], acc[i][j]);
    };

    // Per step kt (A stage kt % 2, weight stage kt % 3), blocks issued:
    //   sub-steps 0, 1, 2: W(kt+2) 0..2, 3..5, 6..7 into the weight stage step
    //   kt-1 freed;
    //   barrier (A(kt+1) and W(kt+1) complete: only the 8 newest loads, all of
    //   W(kt+2), may still be in flight);
    //   sub-step 3: A(kt+2) 0..7 into the A stage step kt freed.
    // prologue: A(0), W(0), W(1) whole, then A(1) (the sub-step-3 share of step -1)
    {
      const u32x4 a0 = kdescA(0), b0 = kdescB(0), b1 = kdescB(1), a1 = kdescA(1);
#pragma unroll
      for (int p = 0; p < PA_; ++p) dmaA(p, 0, koffA(0), a0);
#pragma unroll
      for (int p = 0; p < PB_; ++p) dmaB(p, 0, koff(0), b0);
#pragma unroll
      for (int p = 0; p < PB_; ++p) dmaB(p, 1, koff(1), b1);
      wait_vm<PB_>();
      __syncthreads();
#pragma unroll
      for (int r = 0; r < NR; ++r) frag(0, 0, 0, 0, r);
#pragma unroll
      for (int p = 0; p < PA_; ++p) dmaA(p, 1, koffA(1), a1);
    }

    // one K step; the stage indices are compile-time (the loop runs six steps
    // per iteration: the A stages repeat every 2 steps, the weight stages every 3)
    auto step = [&](int kt, auto U, auto WC) {
      constexpr int u = decltype(U)::value, wcur = decltype(WC)::value;
      constexpr int w1 = (wcur + 1) % 3, w2 = (wcur + 2) % 3;
      const int k2 = koff(kt + 2), k2a = koffA(kt + 2);
      const u32x4 dA2 = kdescA(kt + 2), dB2 = kdescB(kt + 2);
#pragma unroll
      for (int kk = 0; kk < KS - 1; ++kk) {
        int rd = 0, qb = BS0[kk];
        const int qbe = BS0[kk + 1];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          mfma1(kk & 1, m);
          if (rd < NR) frag(u, wcur, kk + 1, (kk + 1) & 1, rd++);
          if ((m & 1) && qb < qbe) dmaB(qb++, w2, k2, dB2);
          __builtin_amdgcn_sched_barrier(0);
        }
        while (rd < NR) frag(u, wcur, kk + 1, (kk + 1) & 1, rd++);
        while (qb < qbe) dmaB(qb++, w2, k2, dB2);
        __builtin_amdgcn_sched_barrier(0);
      }
      wait_vm<PB_>();
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      int rd = 0, qa = 0;
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        mfma1((KS - 1) & 1, m);
        if (rd < NR) frag(u ^ 1, w1, 0, KS & 1, rd++);
        if ((m & 1) && qa < PA_) dmaA(qa++, u, k2a, dA2);
        __builtin_amdgcn_sched_barrier(0);
      }
      while (rd < NR) frag(u ^ 1, w1, 0, KS & 1, rd++);
      while (qa < PA_) dmaA(qa++, u, k2a, dA2);
      __builtin_amdgcn_sched_barrier(0);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    int kt = 0;
    for (; kt + 6 <= nk; kt += 6) {
      step(kt, I0{}, I0{});
      step(kt + 1, I1{}, I1{});
      step(kt + 2, I0{}, I2{});
      step(kt + 3, I1{}, I0{});
      step(kt + 4, I0{}, I1{});
      step(kt + 5, I1{}, I2{});
    }
    // the remaining steps (kt is a multiple of 6 here)
    if (kt < nk) step(kt, I0{}, I0{});
    if (kt + 1 < nk) step(kt + 1, I1{}, I1{});
    if (kt + 2 < nk) step(kt + 2, I0{}, I2{});
    if (kt + 3 < nk) step(kt + 3, I1{}, I0{});
    if (kt + 4 < nk) step(kt + 4, I0{}, I1{});
    // no load may still be writing LDS when an epilogue reuses it
    wait_vm<0>();
  };
  // ---- direct-to-LDS main loop (bf16, 64-row tiles) -------------------------
  // Four stages of 64 A rows and 256 weight rows, 128 bytes per row, swizzled;
  // a stage's 40 blocks of 1 KiB go to wave w as blocks 4p + w.  Step kt + 3 is
  // fetched during step kt (3, 3, 2 blocks in sub-steps 0-2 and 2 after the
  // barrier) into the stage step kt - 1 freed, so each load has about three of
  // these short steps to land.
  auto dtl64_main_loop = [&]() {
    constexpr int SB = (BM + kTileN) * 128;
    constexpr int PW = (BM + kTileN) / 32;  // blocks per wave per step
    constexpr int D[5] = {0, 3, 6, 8, PW};  // blocks issued up to the end of sub-steps 0, 1, 2, 3
    static_assert(!kDTL64 || PW == 10, "issue pattern assumes 10 blocks per wave");
    const int rb_ = static_cast<int>(row_b);
    const u32x4 da = dma_rsrc(A, (gat ? g.a_n : static_cast<int64_t>(m_valid)) * row_b);
    const u32x4 db0 = dma_rsrc(static_cast<const T*>(g.B0) + wofs, static_cast<int64_t>(n_valid) * row_b);
    const u32x4 db1 = NMAT > 1 ? dma_rsrc(static_cast<const T*>(g.B1) + wofs, static_cast<int64_t>(n_valid) * row_b) : db0;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    int doff[PW];
#pragma unroll
    for (int p = 0; p < PW; ++p) {
      const int row = 8 * (4 * p + wv) + (lane >> 3);  // stage row: A rows, then weight rows
      int src = row < BM ? row : row - BM;
      if (NMAT == 2 && row >= BM + 128) src -= 128;
      doff[p] = ((gat && row < BM) ? gather_off(row) : src * rb_) + (((lane & 7) ^ swz(row)) << 4);
    }
    const unsigned lds0 = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(reinterpret_cast<uintptr_t>(lds)));
    // block 4p + w of a stage: A for p < BM / 32, then gate (or the only) weight
    // rows, then up rows; which one is fixed by p alone
    const int nk = K / 64;
    auto koff = [&](int kt) { return kt < nk ? kt * 128 : 0x7ffff000; };
    // a gathered A reloads step 0's rows past the last step (never consumed)
    auto dma = [&](int p, int st, int kt) {
      const unsigned dst = lds0 + st * SB + (4 * p + wv) * 1024;
      if (4 * p < BM / 8) load_lds(da, doff[p] + (gat ? (kt < nk ? kt * 128 : 0) : koff(kt)), dst);
      else if (NMAT == 1 || 4 * p < BM / 8 + 16) load_lds_hint<WNT>(db0, doff[p] + koff(kt), dst);
      else load_lds_hint<WNT>(db1, doff[p] + koff(kt), dst);
    };
    const int sw = swz(lr);
    const int a_rd2 = (wm * (BM / WM) + lr) * 128;
    int b_rd2[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) b_rd2[j] = (BM + brow(j) + lr) * 128;
    int kofs[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) kofs[kk] = ((2 * kk + lg) ^ sw) << 4;
    auto frag = [&](int st, int kk, int buf, int r) {
      const char* sb = lds + st * SB;
      if (r >= 1 && r <= TN) fb[buf][r - 1] = *reinterpret_cast<const Frag*>(sb + b_rd2[r - 1] + kofs[kk]);
      else {
        const int i = r == 0 ? 0 : r - TN;
        fa[buf][i] = *reinterpret_cast<const Frag*>(sb + a_rd2 + i * 32 * 128 + kofs[kk]);
      }
    };
    auto mfma1 = [&](int buf, int m) {
      const int i = m / TN, j = m % TN;
      acc[i][j] = mma(fb[buf][j], fa[buf][i], acc[i][j]);
    };
    // prologue: steps 0, 1, 2 in flight, step 0 published
#pragma unroll
    for (int st = 0; st < 3; ++st)
#pragma unroll
      for (int p = 0; p < PW; ++p) dma(p, st, st);
    wait_vm<2 * PW>();
    __syncthreads();
#pragma unroll
    for (int r = 0; r < NR; ++r) frag(0, 0, 0, r);
    // one K step; its stage index is compile-time (the loop runs four steps per
    // iteration, one per stage)
    auto step = [&](int kt, auto ST) {
      constexpr int st0 = decltype(ST)::value;
      constexpr int st1 = (st0 + 1) & 3, st3 = (st0 + 3) & 3;
      const int k3 = kt + 3;  // the step whose loads this step issues
#pragma unroll
      for (int kk = 0; kk < KS - 1; ++kk) {
        int rd = 0, dq = D[kk];
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          mfma1(kk & 1, m);
          if (rd < NR) frag(st0, kk + 1, (kk + 1) & 1, rd++);
          if (dq < D[kk + 1]) dma(dq++, st3, k3);
          __builtin_amdgcn_sched_barrier(0);
        }
        while (rd < NR) frag(st0, kk + 1, (kk + 1) & 1, rd++);
        while (dq < D[kk + 1]) dma(dq++, st3, k3);
        __builtin_amdgcn_sched_barrier(0);
      }
      // step kt + 1 has landed: the newer loads are step kt + 2's (issued during
      // step kt - 1) and the 8 of step kt + 3 issued so far
      wait_vm<PW + 8>();
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      int rd = 0, dq = D[3];
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        mfma1((KS - 1) & 1, m);
        if (rd < NR) frag(st1, 0, KS & 1, rd++);
        if (dq < D[4]) dma(dq++, st3, k3);
        __builtin_amdgcn_sched_barrier(0);
      }
      while (rd < NR) frag(st1, 0, KS & 1, rd++);
      while (dq < D[4]) dma(dq++, st3, k3);
      __builtin_amdgcn_sched_barrier(0);
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using S2 = std::integral_constant<int, 2>;
    using S3 = std::integral_constant<int, 3>;
    int kt = 0;
    for (; kt + 4 <= nk; kt += 4) {
      step(kt, S0{});
      step(kt + 1, S1{});
      step(kt + 2, S2{});
      step(kt + 3, S3{});
    }
    if (kt < nk) step(kt, S0{});
    if (kt + 1 < nk) step(kt + 1, S1{});
    if (kt + 2 < nk) step(kt + 2, S2{});
    // no load may still be writing LDS when an epilogue reuses it
    wait_vm<0>();
  };
  if constexpr (kDTL) {
    dtl_main_loop();
  } else if constexpr (kDTL64) {
    dtl64_main_loop();
  } else {
  const int nk = K / BK;
  // register stage (kt & 1) ^ 1 holds step kt + 1 when NST == 2
  // unconditional, step 1's loads older than step 2's as in the loop: the wait
  // before each LDS write then covers only the loads issued NST steps earlier
  issue(0, 0, nk);
  stash(0);
  issue(NST - 1, 1, nk);
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (NST == 2) issue(0, 2, nk);
  __syncthreads();
  frags(lds, 0, 0);
  auto step = [&](int kt, auto parity) {
    constexpr int W = NST == 2 ? (decltype(parity)::value ^ 1) : 0;
    const char* sb = lds + (kt & 1) * kStageBytes;
    char* wb = lds + ((kt + 1) & 1) * kStageBytes + loff;
    // past the last step the offset is out of range: the loads return zeros
    // without touching memory
    const int o2 = (kt + 1 + NST < nk) ? goff + (kt + 1 + NST) * 128 : 0x7ffff000;
    const int ao2 = (kt + 1 + NST < nk) ? (kt + 1 + NST) * 128 : 0;
    // sub-steps 0 .. KS-2: MFMAs + next fragments + LDS writes of step kt+1 + loads of step kt+1+NST
#pragma unroll
    for (int kk = 0; kk < KS - 1; ++kk) {
      constexpr int PER = (P + KS - 2) / (KS - 1);
      frags(sb, kk + 1, (kk + 1) & 1);
      mfmas(kk & 1);
      int nw = 0;
#pragma unroll
      for (int p = kk * PER; p < (kk + 1) * PER && p < P; ++p) {
        *reinterpret_cast<uint4*>(wb + p * 32 * kRowBytes) = st[W][p];
        issue_one(W, p, o2, ao2);
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
  };
  if constexpr (NST == 1) {
    for (int kt = 0; kt < nk; ++kt) step(kt, std::integral_constant<int, 0>{});
  } else {
    int kt = 0;
    for (; kt + 1 < nk; kt += 2) {
      step(kt, std::integral_constant<int, 0>{});
      step(kt + 1, std::integral_constant<int, 1>{});
    }
    if (kt < nk) step(kt, std::integral_constant<int, 0>{});
  }
  }

  // ---- epilogues with heavy per-element math: stage the fp32 accumulators
  // through LDS, BM/WM rows at a time, then let every thread walk a few
  // columns of the tile (row-contiguous, coalesced reads of d_h and stores of
  // the results).  Keeps the register epilogue small enough to stay unrolled.
  if constexpr (!kWgrad && EPI == kEpiSwiGLUGrad) {
    // the recompute of g | u with the SwiGLU gradient: g and u of an output
    // column sit CW / 2 stage columns apart; thread (ty, tx) walks output
    // columns 4 tx .. 4 tx + 3 (of NSUB = 128) over rows ty, ty + 8, ...
    static_assert(NMAT == 2, "g and u come from the two weight matrices");
    constexpr int RH = BM / WM;
    constexpr int kPitch = kTileN + 4;
    static_assert(RH * kPitch * 4 <= kLdsBytes, "staging tile must fit in LDS");
    float* stage = reinterpret_cast<float*>(lds);
    __syncthreads();  // every wave is done with the operand stages
#pragma unroll
    for (int h = 0; h < WM; ++h) {
      if (wm == h) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<float4*>(stage + (i * 32 + lr) * kPitch + wn * CW + j * 32 + 8 * q + 4 * lg) =
                  make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
      }
      __syncthreads();
      const int tx = tid & 31, ty = tid >> 5;
      const int oc = 4 * tx;
      const int gc = (oc / (CW / 2)) * CW + oc % (CW / 2);  // stage column of g; u is CW / 2 further
      const int col = n0 + oc;
      T* __restrict__ C = static_cast<T*>(g.C);
      T* __restrict__ C2 = static_cast<T*>(g.C2);
      const float* __restrict__ aux = g.aux;
      const int rows = min(RH, m_valid - h * RH);
      if (col < N) {
        for (int nb = ty; nb < rows; nb += 32) {
          float4 gv[4], uv[4], dv[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {   // rows nb, nb + 8, nb + 16, nb + 24: loads first
            const int n = min(nb + 8 * u, rows - 1);
            const int64_t row = r0 + h * RH + n;
            gv[u] = *reinterpret_cast<const float4*>(stage + n * kPitch + gc);
            uv[u] = *reinterpret_cast<const float4*>(stage + n * kPitch + gc + CW / 2);
            dv[u] = *reinterpret_cast<const float4*>(aux + row * N + col);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (nb + 8 * u >= rows) break;
            const int64_t row = r0 + h * RH + nb + 8 * u;
            float o0[4], o1[4], hv[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              // d_g = d_h * u * silu'(g), d_u = d_h * silu(g), silu'(g) = s (1 + g (1 - s)),
              // with the sigmoid s the forward's activation uses (one exp2 and one
              // reciprocal per element, shared with h)
              const float gt = (&gv[u].x)[c], up = (&uv[u].x)[c], av = (&dv[u].x)[c];
              const float sg = __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(gt * -1.4426950408889634f));
              o0[c] = av * up * (sg * (1.f + gt * (1.f - sg)));
              o1[c] = av * (gt * sg);
              hv[c] = swiglu_h(gt, up);
            }
            const int64_t o = row * 2 * N + col;
            if constexpr (kBf16) {
              *reinterpret_cast<uint2*>(C + o) =
                  make_uint2(f32_to_bf16_bits(o0[0]) | (f32_to_bf16_bits(o0[1]) << 16),
                             f32_to_bf16_bits(o0[2]) | (f32_to_bf16_bits(o0[3]) << 16));
              *reinterpret_cast<uint2*>(C + o + N) =
                  make_uint2(f32_to_bf16_bits(o1[0]) | (f32_to_bf16_bits(o1[1]) << 16),
                             f32_to_bf16_bits(o1[2]) | (f32_to_bf16_bits(o1[3]) << 16));
              *reinterpret_cast<uint2*>(C2 + row * N + col) =
                  make_uint2(f32_to_bf16_bits(hv[0]) | (f32_to_bf16_bits(hv[1]) << 16),
                             f32_to_bf16_bits(hv[2]) | (f32_to_bf16_bits(hv[3]) << 16));
            } else {
              *reinterpret_cast<float4*>(C + o) = make_float4(o0[0], o0[1], o0[2], o0[3]);
              *reinterpret_cast<float4*>(C + o + N) = make_float4(o1[0], o1[1], o1[2], o1[3]);
              *reinterpret_cast<float4*>(C2 + row * N + col) = make_float4(hv[0], hv[1], hv[2], hv[3]);
            }
          }
        }
      }
      __syncthreads();
    }
    return;
  }

  // (the fp32 store takes the same path: its 16-byte stores then cover whole
  // 1 KiB rows instead of 32 bytes in each of 32 rows)
  if constexpr (!kWgrad && (EPI == kEpiGELU || EPI == kEpiGELUGrad || EPI == kEpiStoreF32)) {
    static_assert(NMAT == 1, "staged epilogues take one weight matrix");
    constexpr int RH = BM / WM;  // rows staged per round
    constexpr int kPitch = kTileN + 4;  // floats per staged row (padded: rows start 4 banks apart)
    static_assert(RH * kPitch * 4 <= kLdsBytes, "staging tile must fit in LDS");
    float* stage = reinterpret_cast<float*>(lds);
    __syncthreads();  // every wave is done with the operand stages
#pragma unroll
    for (int h = 0; h < WM; ++h) {
      if (wm == h) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              *reinterpret_cast<float4*>(stage + (i * 32 + lr) * kPitch + wn * CW + j * 32 + 8 * q + 4 * lg) =
                  make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
      }
      __syncthreads();
      // thread (ty, tx): columns 4 tx .. 4 tx + 3 of rows ty, ty + 4, ... (N is a
      // multiple of 64, so a group of four is wholly inside or outside)
      const int tx = tid & 63, ty = tid >> 6;
      const int col = n0 + 4 * tx;
      T* __restrict__ C = static_cast<T*>(g.C);
      const float* __restrict__ aux = g.aux;
      const int rows = min(RH, m_valid - h * RH);
      if (col < N) {
        for (int nb = ty; nb < rows; nb += 16) {
          float4 a[4], p0[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {   // rows nb, nb + 4, nb + 8, nb + 12: loads first
            const int n = min(nb + 4 * u, rows - 1);
            const int64_t row = r0 + h * RH + n;
            a[u] = *reinterpret_cast<const float4*>(stage + n * kPitch + 4 * tx);
            if constexpr (EPI == kEpiGELUGrad) p0[u] = *reinterpret_cast<const float4*>(aux + row * N + col);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (nb + 4 * u >= rows) break;
            const int64_t row = r0 + h * RH + nb + 4 * u;
            const float av[4] = {a[u].x, a[u].y, a[u].z, a[u].w};
            float o0[4], o1[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              if constexpr (EPI == kEpiStoreF32) {
                o0[c] = av[c];
              } else if constexpr (EPI == kEpiGELU) {
                o0[c] = gelu_h(av[c]);
              } else {
                // the recompute of z with the GELU gradient: d_z = d_h (Phi(z) + z phi(z))
                // from the read d_h, and h = gelu(z)
                const float z = av[c], dh = (&p0[u].x)[c];
                o0[c] = dh * (0.5f * (1.f + erff(z * 0.70710678118654752f)) +
                              z * expf(-0.5f * z * z) * 0.39894228040143268f);
                o1[c] = gelu_h(z);
              }
            }
            const int64_t o = row * N + col;
            if constexpr (EPI == kEpiStoreF32) {
              *reinterpret_cast<float4*>(static_cast<float*>(g.C) + o) = make_float4(o0[0], o0[1], o0[2], o0[3]);
            } else if constexpr (kBf16) {
              *reinterpret_cast<uint2*>(C + o) =
                  make_uint2(f32_to_bf16_bits(o0[0]) | (f32_to_bf16_bits(o0[1]) << 16),
                             f32_to_bf16_bits(o0[2]) | (f32_to_bf16_bits(o0[3]) << 16));
              if constexpr (EPI == kEpiGELUGrad)
                *reinterpret_cast<uint2*>(static_cast<T*>(g.C2) + o) =
                    make_uint2(f32_to_bf16_bits(o1[0]) | (f32_to_bf16_bits(o1[1]) << 16),
                               f32_to_bf16_bits(o1[2]) | (f32_to_bf16_bits(o1[3]) << 16));
            } else {
              *reinterpret_cast<float4*>(C + o) = make_float4(o0[0], o0[1], o0[2], o0[3]);
              if constexpr (EPI == kEpiGELUGrad)
                *reinterpret_cast<float4*>(static_cast<T*>(g.C2) + o) = make_float4(o1[0], o1[1], o1[2], o1[3]);
            }
          }
        }
      }
      __syncthreads();
    }
    return;
  }

  // ---- epilogue: the weight fragment is the MFMA's first operand, so lane
  // (lr, lg) of a 32 x 32 tile holds row lr and columns 8 q + 4 lg + c for
  // element 4 q + c: four adjacent outputs, stored with one 8- or 16-byte write
  constexpr int JO = NMAT == 2 ? TN / 2 : TN;  // output column subtiles per wave
  // bf16 outputs of a tall tile: each 8-byte group goes to an LDS copy of
  // the output tile first (rows of NSUB values, 16-byte chunk c of row r at
  // chunk c ^ (r mod chunks): conflict-free for the 32 rows a group write
  // spans), then whole rows leave with 16 bytes per lane, one row segment of
  // 256 or 512 contiguous bytes per 16 or 32 lanes.  Written straight from
  // the accumulators, one 8-byte write covers 16 bytes of each of 32 rows.
  if constexpr (kBf16 && (EPI == kEpiSwiGLU || EPI == kEpiStore) && BM >= kStagedStoreMinBM) {
    constexpr int RB = NSUB * 2;   // bytes per staged row
    constexpr int CH = NSUB / 8;   // 16-byte chunks per row
    static_assert(BM * RB <= kGemmLdsBytes, "staged output tile must fit in LDS");
    __syncthreads();  // every wave is done with the operand stages
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int srow = wm * (BM / WM) + i * 32 + lr;
      if (srow >= m_valid) continue;
#pragma unroll
      for (int j = 0; j < JO; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int cw = (NMAT == 2 ? wn * (CW / 2) : wn * CW) + j * 32 + 8 * q;  // first column of the chunk
          float v[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            v[c] = acc[i][j][4 * q + c];
            if constexpr (EPI == kEpiSwiGLU) v[c] = swiglu_h(v[c], acc[i][j + TN / 2][4 * q + c]);
          }
          store4(reinterpret_cast<uint16_t*>(lds + srow * RB + (((cw >> 3) ^ (srow & (CH - 1))) << 4) + 8 * lg), v);
        }
      }
    }
    __syncthreads();
    const int ch = tid % CH;
    const int col = n0 + 8 * ch;
    if (col < N) {  // N is a multiple of 64: a chunk is wholly in or out
      for (int r = tid / CH; r < m_valid; r += 256 / CH) {
        const int64_t row = r0 + r;
        T* Cr;
        if constexpr (kWgrad)  // weight gradients: rows below c_split to C, the others to C2
          Cr = row < g.c_split
                   ? static_cast<T*>(g.C) + (static_cast<int64_t>(e) * g.c_split + row) * N
                   : static_cast<T*>(g.C2) + (static_cast<int64_t>(e) * (g.Mw - g.c_split) + row - g.c_split) * N;
        else
          Cr = static_cast<T*>(g.C) + row * N;
        *reinterpret_cast<uint4*>(Cr + col) = *reinterpret_cast<const uint4*>(lds + r * RB + ((ch ^ (r & (CH - 1))) << 4));
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int lrow_out = wm * (BM / WM) + i * 32 + lr;
    if (lrow_out >= m_valid) continue;
    const int64_t row = r0 + lrow_out;
#pragma unroll
    for (int j = 0; j < JO; ++j) {
      const int cb = n0 + (NMAT == 2 ? wn * (CW / 2) : wn * CW) + j * 32;
      if (cb >= N) continue;  // N is a multiple of 64: whole 32-column blocks are in or out
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = cb + 8 * q + 4 * lg;
        float v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          v[c] = acc[i][j][4 * q + c];
          if constexpr (EPI == kEpiSwiGLU) v[c] = swiglu_h(v[c], acc[i][j + TN / 2][4 * q + c]);
        }
        if constexpr (kWgrad) {
          T* C = row < g.c_split
                     ? static_cast<T*>(g.C) + (static_cast<int64_t>(e) * g.c_split + row) * N
                     : static_cast<T*>(g.C2) + (static_cast<int64_t>(e) * (g.Mw - g.c_split) + row - g.c_split) * N;
          store4(C + col, v);
        } else if constexpr (EPI == kEpiStoreF32) {
          store4(static_cast<float*>(g.C) + row * N + col, v);
        } else {
          store4(static_cast<T*>(g.C) + row * N + col, v);
        }
      }
    }
  }
}


template <bool kBf16, int NMAT, int EPI, int BM, int WM, bool kWgrad = false, int KM = 0>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_kernel(GemmArgs g) {
  static_assert(gemm_lds_bytes<kBf16, NMAT, EPI, BM, WM, kWgrad>() <= kGemmLdsBytes, "LDS");
  gemm_tile<kBf16, NMAT, EPI, BM, WM, kWgrad, KM>(g, static_cast<int>(blockIdx.x));
}

// 128-row tiles exist for bf16 operands with a register epilogue (the staged
// GELU epilogue needs a 256-column staging tile of 128 rows that does not fit).
template <bool kBf16, int EPI>
constexpr bool kHasMidTiles = kBf16 && (EPI == kEpiSwiGLU || EPI == kEpiStore);

// A 256-row tile table, a 128-row one and a 64-row one in one launch.  Block b
// runs on XCD b mod 8 (the hardware deals blocks to the XCDs in turn), and each
// table gives XCD x a contiguous share of its tiles (gemm_tile's raster).
//
// Fixed schedule (big.steal null, or a launch of fewer than kStealMinTiles
// tiles): the first round_up(n_big * nt, 8) blocks run the 256-row tiles, the
// next round_up(n_mid * nt, 8) the 128-row tiles (ranges' last tiles of at most
// 128 rows), the blocks after them the 64-row tiles (short ranges and re-listed
// trailing tiles); the roundings keep every block's index congruent to its XCD
// in each part.  The shorter tiles are dispatched last and so fill the CUs
// that the last round of 256-row tiles leaves idle.  Blocks past all exit.
//
// Balanced tail (big.steal set): the XCDs run at different clocks under load
// (per-block timestamps: up to 8% apart on one chip), so equal shares end at
// different times and the launch waits for the slowest XCD.  Each XCD's own
// blocks run the first share(256-row) - kStealBig of its 256-row tiles by
// index; its remaining tiles (those kStealBig, then its 128-row and 64-row
// shares, in that order) form its queue, dealt by an atomic counter to its next
// blocks in turn.  Each XCD gets kStealExtra more blocks than it has tiles;
// a block whose own queue is empty takes the next tile of the other XCDs'
// queues, so a faster XCD takes over the tail of a slower one.  Every queue
// entry is handed out once (the counter's old value); a block that finds all
// eight queues empty sets a ninth word (the queues only ever drain) and exits,
// and the blocks after it exit on reading that word.  No block waits for
// another.
// WNT: weights loaded non-temporally (bf16).
constexpr int kStealStride = 32;        // ints between two XCDs' counters (a 128-byte line each)
constexpr int kStealBig = 32;           // 256-row tiles per XCD in its queue
constexpr int kStealExtra = 32;         // blocks per XCD beyond its own tiles
constexpr int kStealMinTiles = 4 * 256; // smaller launches keep the fixed schedule

__device__ __forceinline__ int xcd_share(int n, int x) { return (n >> 3) + (x < (n & 7) ? 1 : 0); }

// The old value of *ctr after adding add (0: a plain read), by thread 0,
// broadcast to the block through the first word of gemm_lds (no tile has
// started using it).
__device__ __forceinline__ int take_next(int32_t* ctr, int add = 1) {
  int* const word = reinterpret_cast<int*>(gemm_lds);
  __syncthreads();  // every lane has read the previous value
  if (threadIdx.x == 0) *word = atomicAdd(ctr, add);
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(*word);
}

template <bool kBf16, int NMAT, int EPI, bool WNT = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_mixed_kernel(GemmArgs big,
                                                                                                   GemmArgs mid,
                                                                                                   GemmArgs small) {
  static_assert(gemm_lds_bytes<kBf16, NMAT, EPI, 256, 2, false>() <= kGemmLdsBytes, "LDS");
  static_assert(gemm_lds_bytes<kBf16, NMAT, EPI, 64, 1, false>() <= kGemmLdsBytes, "LDS");
  constexpr bool kMid = kHasMidTiles<kBf16, EPI>;
  const int tb = *big.n_tiles * big.n_col_tiles;
  const int tm = kMid ? *mid.n_tiles * mid.n_col_tiles : 0;
  const int ts = *small.n_tiles * small.n_col_tiles;
  const int b = static_cast<int>(blockIdx.x);
  int table, bt;  // 0: 256-row, 1: 128-row, 2: 64-row table; the block index gemm_tile reads in it
  if (big.steal && tb + tm + ts >= kStealMinTiles) {
    const int x = b & 7, j = b >> 3;  // this block's XCD and its place in that XCD's order
    const int D = min(kStealBig, tb >> 3);
    const int fixed = xcd_share(tb, x) - D;
    if (j < fixed) {
      table = 0;
      bt = b;
    } else {
      auto qlen = [&](int y) { return D + xcd_share(tm, y) + xcd_share(ts, y); };
      if (j >= fixed + qlen(x) + kStealExtra) return;
      int y = x, q = take_next(big.steal + x * kStealStride);  // own queue first
      bool got = q < qlen(x);
      if (!got && take_next(big.steal + 8 * kStealStride, 0) == 0) {  // then the others', unless all are empty
        for (int t = 1; t < 8 && !got; ++t) {
          y = (x + t) & 7;
          q = take_next(big.steal + y * kStealStride);
          got = q < qlen(y);
        }
        if (!got && threadIdx.x == 0) atomicExch(big.steal + 8 * kStealStride, 1);
      }
      __syncthreads();  // the broadcast word is read before the tile's stages overwrite it
      if (!got) return;
      // entry q of XCD y's queue, as the block index that maps to it in its table
      if (q < D) {
        table = 0;
        bt = 8 * (xcd_share(tb, y) - D + q) + y;
      } else if (q - D < xcd_share(tm, y)) {
        table = 1;
        bt = 8 * (q - D) + y;
      } else {
        table = 2;
        bt = 8 * (q - D - xcd_share(tm, y)) + y;
      }
    }
  } else {
    const int nb = (tb + 7) & ~7, nm = (tm + 7) & ~7;
    table = b < nb ? 0 : (kMid && b < nb + nm) ? 1 : 2;
    bt = table == 0 ? b : table == 1 ? b - nb : b - nb - nm;
  }
  if (table == 0) {
    gemm_tile<kBf16, NMAT, EPI, 256, 2, false, 0, WNT>(big, bt);
    return;
  }
  if constexpr (kMid) {
    static_assert(gemm_lds_bytes<kBf16, NMAT, EPI, 128, 1, false>() <= kGemmLdsBytes, "LDS");
    if (table == 1) {
      gemm_tile<kBf16, NMAT, EPI, 128, 1, false, 0, WNT>(mid, bt);
      return;
    }
  }
  gemm_tile<kBf16, NMAT, EPI, 64, 1, false, 0, WNT>(small, bt);
}

// Lists the row tiles of the GEMMs.  With `merge`, consecutive slots of one
// expert (its replica chunks) form one row range: on one GPU they share the
// same weights, so tiling the run as a whole avoids a partial tile per chunk
// (each row's result does not depend on its tile).  Per range with n rows:
//   kCover:  ceil(n / BM) tiles from its first row (the last may be partial);
//   kPadded: m_pad / BM tiles for every range with rows, the uniform padded
//            batch (tiles wholly past the range's last row exit as soon as the
//            GEMM reads them).
// A tile records its range's first slot, first row and end row.
enum TileMode { kCover = 0, kPadded = 1 };

// Optional 64-row companion tables of a 256-row cover table, one per GEMM g
// that runs on it (its column-tile count nt[g]; 0 = none), for a launch of
// gemm_mixed_kernel: the 256-row tiles first, then the 64-row tiles, which
// fill the CUs the last round of 256-row tiles leaves idle.
//   * short ranges: a range of at most 64 * rem_tiles rows is listed as
//     64-row tiles (the same in both tables) instead of one mostly empty
//     256-row tile.  Longer ranges keep their partial 256-row tile: it runs in
//     step with the range's other tiles and shares their weight reads in L2,
//     where a faster 64-row tile would fetch the weights again;
//   * last round: the trailing r row tiles of the 256-row table are listed
//     again as 64-row tiles when that shortens the modelled launch (one round
//     of 256 blocks; a 256-row block costs 1, a 64-row block small_cost).
// counts[2g] is the number of 256-row tiles GEMM g runs, counts[2g + 1] the
// number of 64-row tiles in its table ([g * cap, ...)).
struct TileSplit {
  int nt[2];
  int cap;
  int rem_tiles;
  float small_cost;
  int32_t* slot;
  int32_t* row0;
  int32_t* rend;
  int32_t* counts;
  // 128-row tiles for GEMM 0 (mid_rows = 0: none): a range longer than the
  // short ranges whose last 256-row tile would hold at most mid_rows rows lists
  // that tile here instead (at most one per range; counts[4] is their number),
  // and GEMM 0 runs the 256-row table without those tails (alt_*, the same
  // capacity as the main table); GEMM 1 keeps the main table.  counts[5] stays 0
  // (the empty 128-row table of GEMM 1).
  int mid_rows;
  int32_t* mid_slot;
  int32_t* mid_row0;
  int32_t* mid_rend;
  int32_t* alt_slot;
  int32_t* alt_row0;
  int32_t* alt_rend;
  // a mixed launch's per-XCD counters and all-empty word (nine words,
  // kStealStride apart), set to zero here before the launch; null: none
  int32_t* steal;
};
constexpr int kWaveBlocks = 256;  // one block per CU

// Modelled duration, in rounds of 256-row blocks, of a mixed launch with
// `big` 256-row and `small` 64-row blocks dispatched in that order.
__device__ inline float mixed_rounds(int64_t big, int64_t small, float c) {
  const int64_t full = big / kWaveBlocks, rest = big % kWaveBlocks;
  const float floor_ = rest > 0 ? 1.f : (small > 0 ? c : 0.f);
  return static_cast<float>(full) + fmaxf(floor_, (static_cast<float>(rest) + c * small) / kWaveBlocks);
}

__global__ __launch_bounds__(256) void tiles_kernel(const int32_t* __restrict__ slot_off,
                                                    const int32_t* __restrict__ slot_expert,
                                                    const int32_t* __restrict__ n_slots_p, int max_slots, int64_t M,
                                                    int E, int mode, int BM, int m_pad, int merge, int max_tiles,
                                                    int32_t* __restrict__ tile_slot, int32_t* __restrict__ tile_row0,
                                                    int32_t* __restrict__ tile_rend, int32_t* __restrict__ n_tiles,
                                                    TileSplit split, int32_t* __restrict__ check) {
  __shared__ int32_t scan[256], scan2[256], scan3[256];
  __shared__ int32_t carry, carry2, carry3;
  // slot tables of up to kLdsSlots slots are read from LDS: the merge walk over
  // an expert's consecutive slots is a chain of dependent reads
  constexpr int kLdsSlots = 1024;
  __shared__ int32_t se_lds[kLdsSlots], so_lds[kLdsSlots + 1];
  const int tid = threadIdx.x;
  const int n = min(max(*n_slots_p, 0), max_slots);
  const bool companion = split.counts != nullptr && mode == kCover && BM == 256;
  const int rem_tiles = companion ? split.rem_tiles : 0;
  const int mid_rows = companion ? split.mid_rows : 0;
  const bool staged = n <= kLdsSlots;
  if (companion && split.steal != nullptr && tid < 9) atomicExch(split.steal + tid * kStealStride, 0);
  if (staged) {
    for (int i = tid; i < n; i += 256) se_lds[i] = slot_expert[i];
    for (int i = tid; i <= n; i += 256) so_lds[i] = slot_off[i];
  }
  const int32_t* se = staged ? se_lds : slot_expert;
  const int32_t* so = staged ? so_lds : slot_off;
  if (tid == 0) carry = carry2 = carry3 = 0;
  // each GEMM's last (up to) 256 tiles of its 256-row table, for the re-listing
  // below: with one chunk of slots (n <= 256) they are captured as they are
  // written (the totals are known once the chunk's scan is done), else read
  // back from the tables
  __shared__ int32_t last_slot[2][256], last_row0[2][256], last_rend[2][256];
  const bool direct = companion && n <= 256;
  __syncthreads();
  if (check) {
    // the slot table a dispatch writes: slot_off ascending inside [0, M],
    // experts inside [0, E), n_slots inside [0, max_slots]
    bool bad = tid == 0 && (*n_slots_p < 0 || *n_slots_p > max_slots);
    for (int i = tid; i < n; i += 256)
      bad |= so[i] < 0 || so[i] > so[i + 1] || so[i + 1] > M || se[i] < 0 || se[i] >= E;
    raise_check(check, bad, MOE_CHECK_SLOTS);
  }
  for (int c = 0; c < n; c += 256) {
    const int s = c + tid;
    int64_t start = 0, end = 0, cnt = 0, cnt_small = 0, cnt_mid = 0;
    if (s < n && !(merge && s > 0 && se[s] == se[s - 1])) {
      int last = s + 1;  // one past the range's last slot
      if (merge)
        while (last < n && se[last] == se[s]) ++last;
      start = min<int64_t>(max(so[s], 0), M);
      end = min<int64_t>(max(so[last], 0), M);
      const int64_t rows = end > start ? end - start : 0;
      if (mode == kCover) {
        cnt = (rows + BM - 1) / BM;
        if (rows > 0 && rows <= 64 * rem_tiles) {
          cnt = 0;
          cnt_small = (rows + 63) / 64;
        } else if (mid_rows > 0 && rows % BM > 0 && rows % BM <= mid_rows) {
          cnt_mid = 1;  // GEMM 0 runs the range's last tile as one 128-row tile
        }
      } else if (rows > 0) {
        cnt = m_pad / BM;
      }
    }
    scan[tid] = static_cast<int32_t>(cnt);
    scan2[tid] = static_cast<int32_t>(cnt_small);
    scan3[tid] = static_cast<int32_t>(cnt_mid);
    __syncthreads();
    for (int d = 1; d < 256; d <<= 1) {
      const int32_t v = tid >= d ? scan[tid - d] : 0;
      const int32_t v2 = tid >= d ? scan2[tid - d] : 0;
      const int32_t v3 = tid >= d ? scan3[tid - d] : 0;
      __syncthreads();
      scan[tid] += v;
      scan2[tid] += v2;
      scan3[tid] += v3;
      __syncthreads();
    }
    // direct capture: GEMM g's table has tot_g[g] tiles, its last 256 from b0_g[g]
    int tot_g[2] = {0, 0}, b0_g[2] = {0, 0};
    if (direct) {
      tot_g[1] = min(scan[255], max_tiles);
      tot_g[0] = mid_rows > 0 ? max(tot_g[1] - scan3[255], 0) : tot_g[1];
      b0_g[0] = max(tot_g[0] - 256, 0);
      b0_g[1] = max(tot_g[1] - 256, 0);
    }
    const int32_t first = carry + scan[tid] - static_cast<int32_t>(cnt);
    for (int q = 0; q < cnt; ++q) {
      const int j = first + q;
      if (j < max_tiles) {
        const int32_t r0 = static_cast<int32_t>(min<int64_t>(start + static_cast<int64_t>(q) * BM, M));
        tile_slot[j] = s;
        tile_row0[j] = r0;
        tile_rend[j] = static_cast<int32_t>(end);
        for (int g = mid_rows > 0 ? 1 : 0; g < 2; ++g)
          if (direct && j >= b0_g[g] && j < tot_g[g]) {
            last_slot[g][j - b0_g[g]] = s;
            last_row0[g][j - b0_g[g]] = r0;
            last_rend[g][j - b0_g[g]] = static_cast<int32_t>(end);
          }
      }
    }
    const int32_t first2 = carry2 + scan2[tid] - static_cast<int32_t>(cnt_small);
    for (int q = 0; q < cnt_small; ++q) {
      const int j = first2 + q;
      for (int g = 0; g < 2; ++g)
        if (split.nt[g] > 0 && j < split.cap) {
          split.slot[g * split.cap + j] = s;
          split.row0[g * split.cap + j] = static_cast<int32_t>(start + static_cast<int64_t>(q) * 64);
          split.rend[g * split.cap + j] = static_cast<int32_t>(end);
        }
    }
    if (mid_rows > 0) {
      // GEMM 0's table: this range's tiles but the 128-row tail, at the main
      // table's position less the tails listed before it
      const int32_t mid_before = carry3 + scan3[tid] - static_cast<int32_t>(cnt_mid);
      const int64_t cnt_b = cnt - cnt_mid;
      for (int q = 0; q < cnt_b; ++q) {
        const int j = first - mid_before + q;
        if (j < max_tiles) {
          const int32_t r0 = static_cast<int32_t>(min<int64_t>(start + static_cast<int64_t>(q) * BM, M));
          split.alt_slot[j] = s;
          split.alt_row0[j] = r0;
          split.alt_rend[j] = static_cast<int32_t>(end);
          if (direct && j >= b0_g[0] && j < tot_g[0]) {
            last_slot[0][j - b0_g[0]] = s;
            last_row0[0][j - b0_g[0]] = r0;
            last_rend[0][j - b0_g[0]] = static_cast<int32_t>(end);
          }
        }
      }
      if (cnt_mid > 0) {  // at most one per range, at most max_slots in all
        split.mid_slot[mid_before] = s;
        split.mid_row0[mid_before] = static_cast<int32_t>(start + cnt_b * BM);
        split.mid_rend[mid_before] = static_cast<int32_t>(end);
      }
    }
    __syncthreads();
    if (tid == 255) {
      carry += scan[255];
      carry2 += scan2[255];
      carry3 += scan3[255];
    }
    __syncthreads();
  }
  const int total = min(carry, max_tiles);
  if (tid == 0) *n_tiles = total;
  if (!companion) return;
  const int n_rem = min(carry2, split.cap);
  const int n_mid = carry3;
  const int total_g[2] = {mid_rows > 0 ? max(total - n_mid, 0) : total, total};
  if (!direct) {
    // more than one chunk: read the last tiles back (the tables' writes by the
    // other threads are visible after the last barrier)
    for (int g = 0; g < 2; ++g) {
      const int32_t* ts = (g == 0 && mid_rows > 0) ? split.alt_slot : tile_slot;
      const int32_t* tr = (g == 0 && mid_rows > 0) ? split.alt_row0 : tile_row0;
      const int32_t* te = (g == 0 && mid_rows > 0) ? split.alt_rend : tile_rend;
      const int b0 = max(total_g[g] - 256, 0);
      if (b0 + tid < total_g[g]) {
        last_slot[g][tid] = ts[b0 + tid];
        last_row0[g][tid] = tr[b0 + tid];
        last_rend[g][tid] = te[b0 + tid];
      }
    }
    __syncthreads();
  }
  // Per GEMM: re-list its last r row tiles (1 <= r <= r_max) as 64-row tiles
  // where the modelled launch is shortest; the smallest r of the shortest.
  // Candidate r is evaluated by lane / thread r - 1: rows(r) = 64-row tiles of
  // the last r tiles (an inclusive scan), valid while the companion table has
  // room for them.  The order key of a candidate is its modelled rounds (a
  // non-negative float orders as its bits), then r.  With r_max <= 64 (at least
  // 4 column tiles) wave g plans GEMM g with shuffles, the two at once;
  // otherwise the block plans them one after the other.
  __shared__ int32_t rows_s[256];
  __shared__ unsigned long long best_key[4];
  const float c = split.small_cost;
  const int lane = tid & 63, wv = tid >> 6;
  int r_max_g[2], tail_g[2];
  for (int g = 0; g < 2; ++g) {
    const int nt = split.nt[g];
    // trailing row tiles of at most one round of blocks (and all staged)
    r_max_g[g] = nt > 0 ? min(min(total_g[g], 256), (kWaveBlocks + nt - 1) / nt) : 0;
    // GEMM 0's 128-row tiles and the short-range 64-row tiles run after the
    // 256-row tiles, both modelled at cost c
    tail_g[g] = n_rem + (g == 0 ? n_mid : 0);
  }
  auto cand_key = [&](int g, int r, int rows) {
    const int nt = split.nt[g], tot = total_g[g];
    const int64_t tail = static_cast<int64_t>(tail_g[g]) * nt;
    float e = __int_as_float(0x7f800000);
    if (r == 0) e = mixed_rounds(static_cast<int64_t>(tot) * nt, tail, c);
    else if (r <= r_max_g[g] && n_rem + rows <= split.cap)
      e = mixed_rounds(static_cast<int64_t>(tot - r) * nt, tail + static_cast<int64_t>(rows) * nt, c);
    return (static_cast<unsigned long long>(__float_as_uint(e)) << 32) | static_cast<unsigned>(r);
  };
  auto own_rows = [&](int g, int r) {
    const int t = total_g[g] - r - max(total_g[g] - 256, 0);
    return r <= r_max_g[g] ? (min(BM, last_rend[g][t] - last_row0[g][t]) + 63) / 64 : 0;
  };
  // tile total_g[g] - r (r <= best_r) goes after the re-listed tiles before it
  auto relist = [&](int g, int r, int rows, int best_rows) {
    const int t = total_g[g] - r - max(total_g[g] - 256, 0);
    int small = n_rem + best_rows - rows;
    const int end = min(last_row0[g][t] + BM, last_rend[g][t]);
    for (int row = last_row0[g][t]; row < end; row += 64) {
      split.slot[g * split.cap + small] = last_slot[g][t];
      split.row0[g * split.cap + small] = row;
      split.rend[g * split.cap + small] = last_rend[g][t];
      ++small;
    }
  };
  if (r_max_g[0] <= 64 && r_max_g[1] <= 64) {
    if (wv < 2) {
      const int g = wv, r = lane + 1;
      int best_r = 0, best_rows = 0;
      if (split.nt[g] > 0) {
        int rows = own_rows(g, r);
        for (int d = 1; d < 64; d <<= 1) {
          const int v = __shfl_up(rows, d);
          if (lane >= d) rows += v;
        }
        unsigned long long key = cand_key(g, r, rows);
        if (lane == 0) {
          const unsigned long long k0 = cand_key(g, 0, 0);
          key = k0 < key ? k0 : key;
        }
        for (int off = 32; off >= 1; off >>= 1) {
          const unsigned long long o = __shfl_xor(key, off);
          key = o < key ? o : key;
        }
        best_r = static_cast<int>(key & 0xffffffffu);
        best_rows = __shfl(rows, best_r > 0 ? best_r - 1 : 0);
        if (best_r == 0) best_rows = 0;
        if (r <= best_r) relist(g, r, rows, best_rows);
      }
      if (lane == 0) {
        split.counts[2 * g] = total_g[g] - best_r;
        split.counts[2 * g + 1] = n_rem + best_rows;
      }
    }
  } else {
    for (int g = 0; g < 2; ++g) {
      int best_r = 0, best_rows = 0;
      if (split.nt[g] > 0) {
        const int r = tid + 1;
        rows_s[tid] = own_rows(g, r);
        __syncthreads();
        for (int d = 1; d < 256; d <<= 1) {
          const int32_t v = tid >= d ? rows_s[tid - d] : 0;
          __syncthreads();
          rows_s[tid] += v;
          __syncthreads();
        }
        const int rows = rows_s[tid];
        unsigned long long key = cand_key(g, r, rows);
        if (tid == 0) {
          const unsigned long long k0 = cand_key(g, 0, 0);
          key = k0 < key ? k0 : key;
        }
        for (int off = 32; off >= 1; off >>= 1) {
          const unsigned long long o = __shfl_xor(key, off);
          key = o < key ? o : key;
        }
        if (lane == 0) best_key[wv] = key;
        __syncthreads();
        unsigned long long bk = best_key[0];
        for (int q = 1; q < 4; ++q) bk = best_key[q] < bk ? best_key[q] : bk;
        best_r = static_cast<int>(bk & 0xffffffffu);
        best_rows = best_r > 0 ? rows_s[best_r - 1] : 0;
        if (r <= best_r) relist(g, r, rows, best_rows);
        __syncthreads();
      }
      if (tid == 0) {
        split.counts[2 * g] = total_g[g] - best_r;
        split.counts[2 * g + 1] = n_rem + best_rows;
      }
    }
  }
  if (tid == 0) {
    split.counts[4] = n_mid;
    split.counts[5] = 0;
  }
}

}  // namespace
