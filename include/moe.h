/*
 * moe.h -- C ABI of libmoe_mi355x.so: one Mixture-of-Experts layer's forward
 * pass on one AMD Instinct MI355X (gfx950), as five stream-ordered calls:
 *
 *   moe_route -> moe_stats -> moe_dispatch -> moe_expert_ffn -> moe_combine
 *
 * plus moe_plan_replicas (a replica plan for the next layer from moe_stats'
 * prediction, made before that layer routes), moe_prediction_quality (how
 * well the prediction and the plan matched the routing that followed),
 * moe_stats_load_state (window variants) and moe_backward (the gradients).
 *
 * Sources (page title, section):
 *   [PF]   "PopFetcher: Towards Accelerated Mixture-of-Experts Training Via
 *           Popularity Based Expert-Wise Prefetch (ATC 2025)", wiki summary
 *   [GPS]  "MoE-GPS框架：动态专家复制的负载均衡优化策略", blog
 *   [EPS]  "EPS-MoE: Expert Pipeline Scheduler for Cost-Efficient MoE Inference",
 *           review
 *   [MPMC] "Fast MoE Inference via Predictive Prefetching and Expert
 *           Replication", summary
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked [host].  The caller allocates
 *     and owns every buffer (outputs, workspaces, the statistics state); the
 *     library never allocates or frees device memory and keeps no device state
 *     between calls.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Each
 *     call checks its host-side arguments, enqueues its kernels on `stream` and
 *     returns without waiting, except where a call says otherwise.
 *   - Return value: MOE_OK or a negative moe_status.  Argument errors are
 *     reported before anything is enqueued; moe_last_error() then holds a
 *     message for the calling thread.  Nothing throws across the ABI.
 *   - Arrays are row-major and contiguous.  Expert weights use the [out, in]
 *     layout per expert, so the reduction dimension is contiguous for both
 *     operands of every product.
 *   - Kernels never access memory outside the extents given, whatever the
 *     values in index arrays; out-of-range indices are skipped (results for
 *     such inputs are unspecified, but memory-safe).
 *   - Device check.  Each of the five hot-path calls takes `check`, a device
 *     pointer to one int32 word owned (and zeroed) by the caller, or NULL.
 *     When it is not NULL, the call's kernels OR into it one MOE_CHECK_* bit
 *     per kind of invalid input they meet (they still skip such entries), and
 *     moe_check_device_error reads it back.  The word accumulates over calls
 *     until the caller zeroes it again; calls on different streams may share
 *     it.  With NULL no check is made.
 *   - Calls are reentrant.  Two in-flight calls must not share an output,
 *     workspace or statistics state.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = -1, /* null pointer, negative size, k > E, misalignment ... */
    MOE_ERR_UNSUPPORTED = -2, /* valid but outside the library's limits (E > 256, H % 64 ...) */
    MOE_ERR_WORKSPACE = -3,   /* workspace or state smaller than the *_bytes query says */
    MOE_ERR_HIP = -4,         /* a HIP runtime call failed; moe_last_error() has its text */
    MOE_ERR_DEVICE_CHECK = -5 /* moe_check_device_error: the kernels flagged invalid input */
} moe_status;

/* Bits of the device-check word (see the conventions above). */
enum {
    MOE_CHECK_LOGITS = 1,     /* moe_route: a NaN or infinite router logit */
    MOE_CHECK_INDEX = 2,      /* moe_stats, moe_dispatch: an expert index outside [0, E) */
    MOE_CHECK_DUPLICATE = 4,  /* moe_stats, moe_dispatch: one token names the same expert twice */
    MOE_CHECK_COUNTS = 8,     /* moe_dispatch: `counts` differs from the counts of topk_idx */
    MOE_CHECK_REPLICAS = 16,  /* moe_dispatch: a negative replica count, or copies beyond max_slots */
    MOE_CHECK_SLOTS = 32,     /* moe_expert_ffn: slot table not ascending inside [0, M], n_slots
                                 outside [0, max_slots], or an expert outside [0, E) */
    MOE_CHECK_ROWS = 64       /* moe_combine: an inv_pos entry outside [0, M) */
};

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;       /* activations and weights */
typedef enum { MOE_SWIGLU = 0, MOE_GELU = 1 } moe_act;
typedef enum { MOE_GEMM_AUTO = 0, MOE_GEMM_GROUPED = 1, MOE_GEMM_DENSE = 2, MOE_GEMM_GROUPED_SMALL = 3 } moe_gemm_path;

/* ---------------------------------------------------------------- routing
 * moe_route -- top-k softmax gate ([PF] observations and trade-offs: the naive
 * top-k gate; [MPMC] problem statement: softmax routing).
 *   logits    fp32 [T, E]
 *   topk_idx  int32 [T, k] out: the k experts of each token, by logit
 *             descending; equal logits go to the lower expert index; slot 0 is
 *             the top-1.
 *   topk_w    fp32 [T, k] out: softmax probabilities of the kept experts,
 *             renormalised to sum to one (= softmax over the kept logits).
 * Limits: 1 <= E <= 256, 1 <= k <= min(E, 8), 0 <= T, T*k < 2^31.
 * Logits are expected finite; NaN is ordered as -inf (indices stay in range).
 * check: MOE_CHECK_LOGITS for a NaN or infinite logit.
 */
int moe_route(const float* logits, int64_t T, int E, int k, int32_t* topk_idx, float* topk_w,
              int32_t* check, void* stream);

/* ------------------------------------------------------------- statistics
 * Sliding-window routing statistics of a chain of L MoE layers ([PF] method:
 * Routing Information Collector, sliding window s, Eq.(1)-(3); [GPS] 2.1:
 * distribution-only prediction p_i = n_i / N with a sliding-window average).
 *
 * The state is a caller-owned device buffer of moe_stats_state_bytes(L, E,
 * window) bytes holding, per layer, a ring of `window` per-iteration count
 * vectors, per adjacent layer pair a ring of E x E co-occurrence matrices and
 * their running sum over the ring, and a small accumulator.  It is plain
 * memory: a checkpoint is a byte copy.
 * moe_stats_init zeroes it (enqueued on `stream`).
 *
 * moe_stats records layer `layer` of iteration `iter` and reports:
 *   - counts[e]   int32 [E]: tokens routed to e by topk_idx (this iteration);
 *   - p_seq[e]    fp32 [E]: window popularity of `layer`,
 *                 Nw[e] / sum(Nw), Nw = the ring's counts summed ([PF] Eq.(1));
 *   - cond        fp32 [E, E]: Pr(next = b | this = a) for pair (layer,
 *                 layer+1), the pair's windowed co-occurrence with each row
 *                 normalised (zero rows stay zero) ([PF] Eq.(2));
 *   - pred_next   fp32 [E]: predicted popularity of layer+1,
 *                 sum_a p_seq[a] * cond[a, b] ([PF] Eq.(3));
 *   - replicas    int32 [E]: extra copies per expert from this iteration's
 *                 counts: the budget of `replica_budget` copies is handed out
 *                 one at a time to the expert with the largest per-copy load
 *                 counts[e]/(r_e+1) among those still above the mean
 *                 T*k/E per copy (counts[e]*E > T*k*(r_e+1)); ties go to the
 *                 lower index ([GPS] 2.1 duplicate_experts with threshold 1;
 *                 [MPMC] contribution 3: capacity-bounded replication).
 * Recording replaces ring slot iter % window of layer's counts and, when
 * layer > 0, of pair (layer-1, layer)'s co-occurrence (k*k pairs per token,
 * from prev_topk_idx = layer-1's routing of the same tokens).  The outputs are
 * computed after that update, so p_seq covers the last `window` recorded
 * iterations and cond/pred_next, whose pair has not recorded `iter` yet,
 * cover the `window` iterations before it: a causal prediction.
 * Any output pointer may be NULL (not written).  cond and pred_next are not
 * written when layer == L-1.  topk_idx == NULL records nothing and only
 * reports (T, k and prev_topk_idx are then ignored; counts and replicas are
 * not written).
 * Limits: 1 <= E <= 256, 1 <= L, 1 <= window <= 1024, 0 <= layer < L,
 * iter >= 0, window * T * k * k < 2^31, 0 <= replica_budget <= 4096.
 * check: MOE_CHECK_INDEX for an entry of topk_idx or prev_topk_idx outside
 * [0, E) (not counted), MOE_CHECK_DUPLICATE for a token naming one expert
 * twice in topk_idx (counted as often as named).
 */
size_t moe_stats_state_bytes(int L, int E, int window); /* [host] */
int moe_stats_init(void* state, size_t state_bytes, int L, int E, int window, void* stream);
int moe_stats(void* state, size_t state_bytes, int L, int E, int window, int layer, int64_t iter,
              const int32_t* topk_idx, const int32_t* prev_topk_idx, int64_t T, int k,
              int32_t* counts, float* p_seq, float* cond, float* pred_next,
              int replica_budget, int32_t* replicas, int32_t* check, void* stream);

/*
 * moe_stats_load_state -- window variants of layer `layer` after iteration
 * `iter` has been recorded by moe_stats (read-only on the state):
 *   p_decay    fp32 [E] (may be NULL): decayed-window popularity ([GPS] 2.1: a
 *              decay factor on the sliding-window average against drift):
 *              over the m = min(window, iter+1) recorded iterations, age 0 =
 *              `iter`, D[e] = sum_age decay^age * n_e(age) (weights by repeated
 *              multiplication, age order, double), p_decay = D / sum(D)
 *              (0 when the sum is 0); decay = 1 gives p_seq, decay = 0 this
 *              iteration's shares;
 *   anomalous  int32 [E] (may be NULL): 1 where the load of `iter` leaves its
 *              history by more than twice the standard deviation ([GPS] 6.1),
 *              (n_e - mean)^2 > 4 var over the m-1 earlier window iterations;
 *              every expert is flagged while fewer than 2 earlier iterations
 *              exist;
 *   summary    int32 [2] (may be NULL): the number of flagged experts, and 1
 *              if the layer is in a transient state (more than a fifth of its
 *              experts flagged, a chosen fraction) or 0 if stable (the
 *              load-prediction study's transient/stable load states).
 * The ring must hold iterations iter-m+1 .. iter of `layer` (recorded in
 * order).  Limits: those of moe_stats, 0 <= decay <= 1.
 */
int moe_stats_load_state(const void* state, size_t state_bytes, int L, int E, int window, int layer,
                         int64_t iter, double decay, float* p_decay, int32_t* anomalous, int32_t* summary,
                         void* stream);

/* ------------------------------------------------ planning ahead of routing
 * moe_plan_replicas -- replica counts for a layer planned before it routes,
 * from a predicted expert distribution ([PF] method: Eq.(3) predicts the next
 * layer's popularity and the plan acts on it ahead of time; [MPMC]
 * contributions 2-3: replicas placed from predicted activity, within a budget).
 *   pred         fp32 [E]: predicted shares, e.g. moe_stats' pred_next of the
 *                layer before;
 *   total        rows the layer will route (T*k);
 *   pred_counts  int32 [E] out (may be NULL): pred[e] * total in double,
 *                rounded to the nearest integer with halves to even; NaN, zero
 *                or negative shares give 0, values from 2^31 - 1 up clamp there;
 *   replicas     int32 [E] out: the greedy plan moe_stats applies to counts,
 *                applied to pred_counts with their sum standing for T*k.
 * Limits: 1 <= E <= 256, 0 <= total < 2^31, 0 <= replica_budget <= 4096.
 *
 * moe_prediction_quality -- how well a prediction matched the routing that
 * followed and how evenly a replica plan spread its rows ([MPMC] evaluation:
 * prediction accuracy and load balance; [GPS] 2.1: per-copy load near the
 * mean).  Writes fp32 out[4]:
 *   out[0]  total-variation distance 0.5 * sum_e |q_e - a_e| between
 *           q = pred / sum(pred) and the actual shares a = counts / sum(counts)
 *           (1 when either sum is not positive);
 *   out[1]  top-n hit rate |top_n(pred) & top_n(counts)| / n, n = min(top_n, E),
 *           ranking by value descending then index ascending (NaN as -inf);
 *   out[2]  population standard deviation of the per-slot row loads, expert e
 *           with r_e replicas being cut into r_e + 1 chunks as moe_dispatch
 *           cuts it (replicas NULL: one slot per expert; r_e clamped to
 *           [0, 4096]);
 *   out[3]  largest slot load over the mean slot load (0 with no rows).
 * Sums are taken in expert order in double and rounded to fp32 once.
 * Limits: 1 <= E <= 256, top_n >= 1.  Both calls are one small kernel on
 * `stream`; pointers are device pointers.
 */
int moe_plan_replicas(const float* pred, int E, int64_t total, int replica_budget, int32_t* pred_counts,
                      int32_t* replicas, void* stream);
int moe_prediction_quality(const float* pred, const int32_t* counts, int E, const int32_t* replicas, int top_n,
                           float* out, void* stream);

/* --------------------------------------------------------------- dispatch
 * moe_dispatch -- permute tokens into expert/replica-contiguous rows (the
 * token dispatch that precedes the expert computation; [EPS] section 3 and
 * [PF] motivation: the dispatch All-to-All, here a local permute).  With
 * M = T*k rows:
 *   expert_off  int32 [E+1]: exclusive prefix sum of the per-expert counts;
 *               expert e owns rows [expert_off[e], expert_off[e+1]).
 *   perm_src    int32 [M]: source token of each row.  Inside an expert, rows
 *               follow ascending token index (a stable permutation: pairs
 *               (t, i) in ascending t*k + i, so a token naming one expert
 *               twice gets two rows, slot order).
 *   inv_pos     int32 [T, k]: the row holding (t, topk_idx[t, i]).
 *   x_perm      [M, H] in dtype `dt`: x_perm[r] = x[perm_src[r]] (byte copy).
 *               May be NULL (then x may be NULL too): no row is copied, and
 *               moe_expert_ffn gathers the rows from x with perm_src as its
 *               row map; every other output is written the same way.
 *   slot table  replicas[e] extra copies cut expert e's rows into
 *               replicas[e]+1 contiguous chunks in token order, chunk rho
 *               covering [floor(rho*n_e/(r_e+1)), floor((rho+1)*n_e/(r_e+1)))
 *               of the expert's rows ([MPMC] method: replicas of one expert
 *               serve disjoint token subsets).  Slots are expert-major:
 *               slot_expert [max_slots], slot_off [max_slots+1] (slot s owns
 *               rows [slot_off[s], slot_off[s+1])), n_slots [1].  Unused slots
 *               up to max_slots are empty (slot_off = M).  replicas == NULL
 *               means one slot per expert, unless replica_budget > 0.  Copies
 *               beyond max_slots - E are dropped in expert order (the kernel
 *               never writes past max_slots); negative counts are taken as 0.
 *   replica_budget  with replicas == NULL and replica_budget = R > 0, the
 *               dispatch plans the replicas itself from this routing's
 *               counts: the greedy capacity-bounded rule of moe_stats and
 *               moe_plan_replicas ([GPS] section 2.1, [MPMC] method; total =
 *               T*k), the same plan moe_stats writes for these counts.  So
 *               the replicated layer needs no moe_stats before its dispatch,
 *               and the statistics can run beside the rest of the layer.
 *               Needs max_slots >= E + R; 0 with non-NULL replicas.
 *   counts      int32 [E] (may be NULL): moe_stats' counts of this routing.
 *               The offsets come from topk_idx itself (rows are ranked per
 *               block of pairs, which needs the per-block counts anyway);
 *               `counts` is only compared with them (MOE_CHECK_COUNTS).
 *   workspace   at least moe_dispatch_workspace_bytes(T, k, E) bytes
 *               (per-block counts and offsets, per-pair ranks); any contents.
 * Three launches: per block of 512 (token, slot) pairs its counts and each
 * pair's rank among the block's pairs of its expert (wave ballots); one block
 * turning the block counts into offsets, the replica plan (replica_budget)
 * and the slot table; the row copy, which also writes perm_src and inv_pos.
 * Small dispatches (T*k <= 1024 and E <= 64) take one launch instead, one
 * block doing all three steps (plus the row copy when x_perm is given), and
 * leave the workspace untouched; the results are the same.
 * check: MOE_CHECK_INDEX (an index outside [0, E): inv_pos = -1, no row),
 * MOE_CHECK_DUPLICATE, MOE_CHECK_COUNTS, MOE_CHECK_REPLICAS.
 * Limits: 1 <= E <= 256, 1 <= k <= min(E, 8), T*k < 2^31, E <= max_slots,
 * 0 <= replica_budget <= max_slots - E (0 when replicas is given),
 * H*sizeof(dt) % 16 == 0, x and x_perm 16-byte aligned.
 */
size_t moe_dispatch_workspace_bytes(int64_t T, int k, int E); /* [host] */
int moe_dispatch(const void* x, moe_dtype dt, int64_t T, int H, const int32_t* topk_idx, int k, int E,
                 const int32_t* counts, const int32_t* replicas, int replica_budget, int max_slots,
                 void* x_perm, int32_t* perm_src, int32_t* inv_pos, int32_t* expert_off,
                 int32_t* slot_off, int32_t* slot_expert, int32_t* n_slots,
                 void* workspace, size_t workspace_bytes, int32_t* check, void* stream);

/*
 * moe_dispatch_noalloc -- moe_dispatch for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments without the workspace, which is a
 * static 8 MiB device array of the library instead (held by each GPU the
 * library runs on until the process ends; its address is looked up once per
 * device).  Calls no allocating routine.  Limit: moe_dispatch_workspace_bytes(
 * T, k, E) <= 8 MiB (e.g. T*k <= 2^20 pairs at E = 256), else
 * MOE_ERR_WORKSPACE.  Every call on one GPU shares the array: calls that
 * overlap on one GPU (different streams, or threads) race and must be
 * serialised by the caller.  Nothing in it needs clearing between calls (each
 * call writes every word it reads).  Same results as moe_dispatch; the small
 * dispatches that moe_dispatch runs in one block do not touch the array.
 */
int moe_dispatch_noalloc(const void* x, moe_dtype dt, int64_t T, int H, const int32_t* topk_idx, int k, int E,
                         const int32_t* counts, const int32_t* replicas, int replica_budget, int max_slots,
                         void* x_perm, int32_t* perm_src, int32_t* inv_pos, int32_t* expert_off,
                         int32_t* slot_off, int32_t* slot_expert, int32_t* n_slots, int32_t* check, void* stream);

/* ------------------------------------------------------------- expert FFN
 * moe_expert_ffn -- every slot's rows through its expert's FFN ([EPS] section
 * 3: the gate, up and down GEMMs; GroupGemm runs all experts in one kernel,
 * DenseGemm runs a uniform padded batch):
 *   SwiGLU: h = silu(x Wg^T) * (x Wu^T), y = h Wd^T
 *           w_gate, w_up [E, I, H]; w_down [E, H, I]
 *   GELU:   h = gelu(x W1^T) (exact erf form), y = h W2^T
 *           w_gate = W1 [E, I, H]; w_up must be NULL; w_down = W2 [E, H, I]
 * bf16 inputs are multiplied on bf16 MFMA with fp32 accumulation, fp32 inputs
 * on fp32 MFMA; h is rounded to dtype (kept in the workspace), then y.  Each
 * row's result depends only on that row: it is the same whichever slot, tile
 * or path computes it (fixed reduction order, no split-K), so replicated and
 * non-replicated dispatches give bit-identical y_perm.
 *   path  GROUPED: 256-row tiles cover each slot's rows exactly (no host
 *                  sync): the large-batch form.  A slot range of at most 64
 *                  rows runs as one 64-row tile in the same launch, after the
 *                  256-row tiles.
 *         GROUPED_SMALL: 64-row tiles cover each slot's rows exactly (no
 *                  host sync): less padding when slots hold few rows.
 *         DENSE:   every slot with rows is padded to the largest slot's row
 *                  count (rounded up to 64) and the uniform batch runs in
 *                  64-row tiles; tiles wholly in the padding exit at once.
 *                  Reads the slot table back (synchronises `stream`).
 *         AUTO:    reads the slot table back and picks per GEMM the tiling
 *                  with the lowest modelled cost (tile count x per-tile cost,
 *                  a 64-row tile costing 0.55 of a 256-row one, at least one
 *                  wave of 256 CUs per grid), fitted to measured crossovers.
 *         All paths give bit-identical y_perm.  In every path consecutive
 *         slots of one expert (replicas) are tiled as one row range.  Where a
 *         GEMM runs on 256-row tiles whose blocks leave the launch's last
 *         round of the 256 CUs mostly idle, its trailing row tiles are listed
 *         again as 64-row tiles when the same cost model says so (decided on
 *         the device, no host sync).
 *   row_src    NULL: x_perm holds the M rows [M, H].  Otherwise int32 [M]:
 *              x_perm is an [n_src, H] matrix (the tokens x) and row r of the
 *              FFN's input is x_perm[row_src[r]] (moe_dispatch's perm_src):
 *              the gate/up GEMM gathers its operand rows with per-lane
 *              offsets of its direct-to-LDS loads, so a dispatch without the
 *              row copy (x_perm NULL there) feeds the FFN directly.  Entries
 *              outside [0, n_src) read as zero rows.  n_src * H * sizeof(dt)
 *              must stay below 0x7e000000 bytes (MOE_ERR_UNSUPPORTED).
 *   workspace  at least moe_expert_ffn_workspace_bytes(...) bytes: h, the
 *              tile tables and the counters that deal the gate/up launch's
 *              last tiles, all rewritten by every call, so two calls in
 *              flight at once (on different streams) need two workspaces.
 * Limits: dtype F32 or BF16; H and I multiples of 64; E <= max_slots;
 * M <= 2^31 - 1; rows referenced by slot_off lie in [0, M) (rows outside it
 * are clamped away).
 * check: MOE_CHECK_SLOTS.
 */
size_t moe_expert_ffn_workspace_bytes(moe_dtype dt, int64_t M, int H, int I, int max_slots); /* [host] */
int moe_expert_ffn(const void* x_perm, const int32_t* row_src, int64_t n_src, moe_dtype dt, int64_t M, int H, int I,
                   int E, const int32_t* slot_off, const int32_t* slot_expert, const int32_t* n_slots, int max_slots,
                   const void* w_gate, const void* w_up, const void* w_down, moe_act act, moe_gemm_path path,
                   void* y_perm, void* workspace, size_t workspace_bytes, int32_t* check, void* stream);

/*
 * moe_expert_ffn_profiled -- moe_expert_ffn that also records three caller-owned
 * hipEvent_t handles (passed as void*) on `stream`: events[0] right before the
 * gate/up (W1) GEMM launch, events[1] right after it and events[2] right after
 * the down (W2) GEMM, so a profiler can time the two launches on the library's
 * own stream.  events must hold three valid events.  Same results as
 * moe_expert_ffn.
 */
int moe_expert_ffn_profiled(const void* x_perm, const int32_t* row_src, int64_t n_src, moe_dtype dt, int64_t M,
                            int H, int I, int E, const int32_t* slot_off, const int32_t* slot_expert,
                            const int32_t* n_slots, int max_slots, const void* w_gate, const void* w_up,
                            const void* w_down, moe_act act, moe_gemm_path path, void* y_perm, void* workspace,
                            size_t workspace_bytes, int32_t* check, void* const* events, void* stream);

/* ---------------------------------------------------------------- combine
 * moe_combine -- weighted combine back to token order ([EPS] section 3: the
 * LocalReduce that follows the expert computation):
 *   out[t] = sum_{i<k} topk_w[t, i] * y_perm[inv_pos[t, i]]
 * accumulated in fp32 in slot order i = 0..k-1, rounded once to dtype.
 * inv_pos entries outside [0, M) contribute nothing (MOE_CHECK_ROWS).
 * Limits: 1 <= k <= 8, H*sizeof(dt) % 16 == 0, y_perm and out 16-byte aligned.
 */
int moe_combine(const void* y_perm, moe_dtype dt, int64_t M, const int32_t* inv_pos, const float* topk_w,
                int64_t T, int k, int H, void* out, int32_t* check, void* stream);

/* ----------------------------------------------------------- device check
 * moe_check_device_error -- waits for `stream`, then reads the device-check
 * word `check` (see the conventions above).  Returns MOE_OK if it is zero,
 * else MOE_ERR_DEVICE_CHECK with the flagged kinds named in moe_last_error().
 * bits [host] (may be NULL) receives the word.  The word is left as it is.
 * The stated source of the preconditions: softmax routing over finite logits
 * ("Fast MoE Inference via Predictive Prefetching and Expert Replication",
 * problem statement) picking k distinct experts per token ([PF] observations:
 * the top-k gate).
 */
int moe_check_device_error(const int32_t* check, int32_t* bits, void* stream);

/* ----------------------------------------------------------------- backward
 * moe_backward -- gradients of the layer w.r.t. its tokens, router logits and
 * expert weights, given d_out = dLoss/d out (training, as in [PF] method: the
 * backward pass of MoE training with its reverse All-to-All, here local).  The
 * chain rule through the forward above:
 *   dw[t,i]      = <d_out[t], y_perm[inv_pos[t,i]]>            (fp32)
 *   d_logits     fp32 [T, E]: w_j (dw_j - sum_i w_i dw_i) at e = topk_idx[t,j],
 *                0 elsewhere (softmax over the kept logits);
 *   d_y[r]       = w[t,i] d_out[t] for r = inv_pos[t,i]       (dtype);
 *   d_h          = d_y Wd, kept in fp32;
 *   pre-activations g = x Wg^T, u = x Wu^T (GELU: z = x W1^T) recomputed by
 *   the grouped GEMM, whose epilogue meets their fp32 values with d_h:
 *   d_g | d_u    = d_h u silu'(g) | d_h silu(g) (GELU: d_z = d_h gelu'(z)),
 *                rounded to the dtype, and h rebuilt as the forward computes
 *                and rounds it;
 *   d_x[t]       = sum_i d_x_perm[inv_pos[t,i]], d_x_perm = d_g Wg + d_u Wu;
 *   d_w_down[e]  = sum over expert e's rows of d_y^T h ([E, H, I]);
 *   d_w_gate[e], d_w_up[e] = sum over the rows of d_g^T x_perm, d_u^T x_perm
 *                ([E, I, H]; GELU: d_w_gate is d_W1, w_up and d_w_up NULL).
 * Inputs are the forward's own: x_perm and expert_off from moe_dispatch (rows
 * grouped by expert; replica slots do not matter here), y_perm from
 * moe_expert_ffn, topk_idx/topk_w from moe_route, inv_pos from moe_dispatch.
 * All gradients are written whole (experts with no rows get zero weight
 * gradients).  Workspace: moe_backward_workspace_bytes(...) bytes (fp32 d_h,
 * h, transposed weights, expert-padded transposed activations).
 * Limits: those of moe_expert_ffn; T*k < 2^30.
 */
size_t moe_backward_workspace_bytes(moe_dtype dt, int64_t T, int k, int H, int I, int E, moe_act act); /* [host] */
int moe_backward(const void* x_perm, const void* y_perm, moe_dtype dt, int64_t T, int k, int H, int I, int E,
                 const int32_t* topk_idx, const float* topk_w, const int32_t* inv_pos, const int32_t* expert_off,
                 const void* w_gate, const void* w_up, const void* w_down, moe_act act, const void* d_out,
                 void* d_x, float* d_logits, void* d_w_gate, void* d_w_up, void* d_w_down, void* workspace,
                 size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------- errors */
const char* moe_status_string(int status); /* [host] static text */
const char* moe_last_error(void);          /* [host] calling thread's last message */

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
