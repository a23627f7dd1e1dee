"""GPU parity: the HIP path through the C ABI against the CPU oracle, on the same
seeded inputs.  Small shapes are compared element by element (several tiles and
ragged tails); the full workload shapes are compared bit-exactly on every
integer output and on sampled tokens for the floating-point outputs."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_top_amd as moe
import oracle
import synth
from _util import assert_close, f64, from_dev, to_dev

pytestmark = pytest.mark.gpu


def _sync():
    torch.cuda.synchronize()


def _logits(T, E, seed, skew=1.0):
    rng = np.random.default_rng(seed)
    bias = -skew * np.log1p(rng.permutation(E)).astype(np.float32)
    return (rng.standard_normal((T, E)).astype(np.float32) + bias).astype(np.float32)


# ------------------------------------------------------------------ routing
@pytest.mark.parametrize("T,E,k", [(256, 8, 2), (1000, 160, 6), (333, 16, 4), (4097, 32, 2), (77, 5, 3),
                                   (50, 256, 8), (64, 1, 1), (10, 3, 3), (129, 7, 7)])
def test_route_matches_oracle(T, E, k):
    for lg in (_logits(T, E, T + E), synth.tie_logits(T, E)):
        idx, w = moe.moe_route(to_dev(lg), k)
        _sync()
        ridx, rw = oracle.route(lg, k)
        assert np.array_equal(from_dev(idx), ridx)
        assert_close(from_dev(w), rw, "fp32", "topk_w")
        assert np.max(np.abs(from_dev(w) - rw)) <= 2e-6


@pytest.mark.parametrize("name,T", [("mixtral", 8192), ("dsv2", 16384), ("dbrx", 4096), ("popfetcher", 16384)])
def test_route_full_size(name, T):
    cfg = synth.CONFIGS[name].with_T(T)
    lg = synth.logits(cfg, 0, 0)
    idx, w = moe.moe_route(to_dev(lg), cfg.k)
    _sync()
    ridx, rw = oracle.route(lg, cfg.k)
    assert np.array_equal(from_dev(idx), ridx)
    assert_close(from_dev(w), rw, "fp32", "topk_w")


def test_route_empty_batch():
    idx, w = moe.moe_route(torch.empty((0, 8), dtype=torch.float32, device="cuda"), 2)
    _sync()
    assert idx.shape == (0, 2)


# --------------------------------------------------------------- statistics
def _run_stats_chain(cfg, iters, check_every=True):
    """Route + record every layer of every iteration on both sides and compare."""
    L, E, k, win, R = cfg.L, cfg.E, cfg.k, cfg.window, cfg.R
    state = torch.empty(moe.moe_stats_state_bytes(L, E, win), dtype=torch.uint8, device="cuda")
    moe.moe_stats_init(state, L, E, win)
    ost = oracle.WindowStats(L, E, win)
    outs = {n: torch.empty(s, dtype=d, device="cuda") for n, s, d in
            [("counts", E, torch.int32), ("p_seq", E, torch.float32), ("cond", (E, E), torch.float32),
             ("pred", E, torch.float32), ("reps", E, torch.int32)]}
    for it in range(iters):
        prev_o, prev_g = None, None
        for layer in range(L):
            lg = synth.logits(cfg, layer, it, None if prev_o is None else prev_o[:, 0])
            idx_g, _ = moe.moe_route(to_dev(lg), k)
            last = layer + 1 >= L
            moe.moe_stats(state, L, E, win, layer, it, idx_g, prev_g, k, outs["counts"], outs["p_seq"],
                          None if last else outs["cond"], None if last else outs["pred"], R,
                          outs["reps"] if R > 0 else None)
            _sync()
            idx_o, _ = oracle.route(lg, k)
            assert np.array_equal(from_dev(idx_g), idx_o), (it, layer)
            cnt = ost.record(layer, it, idx_o, prev_o)
            if check_every or it == iters - 1:
                assert np.array_equal(from_dev(outs["counts"]), cnt), (it, layer)
                p, P, ph = ost.outputs(layer)
                assert_close(from_dev(outs["p_seq"]), p, "fp32", "p_seq")
                assert np.max(np.abs(from_dev(outs["p_seq"]) - p)) <= 1e-7
                if not last:
                    assert_close(from_dev(outs["cond"]), P, "fp32", "cond")
                    assert np.max(np.abs(from_dev(outs["cond"]) - P)) <= 1e-7
                    assert np.max(np.abs(from_dev(outs["pred"]) - ph)) <= 1e-6
                if R > 0:
                    assert np.array_equal(from_dev(outs["reps"]), oracle.replicas(cnt, cfg.T, k, R))
            prev_o, prev_g = idx_o, idx_g
    return state, ost


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 6, 7, 8])
def test_combine_every_k(dt, k):
    """moe_combine on its own against the oracle's combine (an fp64 sum over the
    k slots, rounded once) for every k: 700 tokens of a ragged row width (H =
    200: 25 bf16 chunks or 50 fp32 chunks of 16 bytes, not a multiple of the
    four chunks a thread takes), random gate weights and rows.  The kernel sums
    in fp32 FMAs in slot order, so an element may differ from the oracle by the
    fp32 chain's error, at most (k + 1) 2^-24 sum_i |w_i y_i| before the output
    rounding (bf16: one unit in the last place of the output on top)."""
    rng = np.random.default_rng(100 + k)
    T, H, M = 700, 200, 1500
    y32 = rng.standard_normal((M, H)).astype(np.float32)
    y = synth.f32_to_bf16_bits(y32) if dt == "bf16" else y32
    yv = f64(y)
    inv = np.stack([rng.choice(M, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), size=T).astype(np.float32)
    got = from_dev(moe.moe_combine(to_dev(y), to_dev(inv), to_dev(w)))
    ref = oracle.combine(y, inv, w)
    g, r = f64(got), f64(ref)
    mag = np.einsum("tk,tkh->th", np.abs(w.astype(np.float64)), np.abs(yv[inv]))
    bound = (k + 1) * 2.0 ** -24 * mag
    if dt == "bf16":  # plus one bf16 unit of the larger magnitude
        bound += 2.0 ** (np.floor(np.log2(np.maximum(np.maximum(np.abs(g), np.abs(r)), 1e-30))) - 7)
    assert np.all(np.abs(g - r) <= bound), float(np.max(np.abs(g - r) - bound))


@pytest.mark.parametrize("k", [2, 3, 8])
def test_combine_skips_rows_outside_y(k):
    """A slot whose row index lies outside [0, M) adds nothing: the output equals
    the combine with that slot given weight 0 on a valid row, bit for bit."""
    rng = np.random.default_rng(7 + k)
    T, H, M = 300, 4096, 900
    y = synth.f32_to_bf16_bits(rng.standard_normal((M, H)).astype(np.float32))
    inv = np.stack([rng.choice(M, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    w = rng.dirichlet(np.ones(k), size=T).astype(np.float32)
    drop = rng.random((T, k)) < 0.25
    inv_bad = np.where(drop, np.where(rng.random((T, k)) < 0.5, -1, M + 5), inv).astype(np.int32)
    w0 = np.where(drop, 0.0, w).astype(np.float32)
    a = from_dev(moe.moe_combine(to_dev(y), to_dev(inv_bad), to_dev(w)))
    b = from_dev(moe.moe_combine(to_dev(y), to_dev(inv), to_dev(w0)))
    assert np.array_equal(a, b)


def test_stats_tiny_chain_window():
    cfg = synth.CONFIGS["tiny"]
    state, ost = _run_stats_chain(cfg, 14)   # wraps the 10-slot ring
    # read-only call after layer 1 recorded the last iteration: the prediction
    # for layer 1 from layer 0 now equals layer 1's own popularity.
    E = cfg.E
    pred = torch.empty(E, dtype=torch.float32, device="cuda")
    p0 = torch.empty(E, dtype=torch.float32, device="cuda")
    moe.moe_stats(state, cfg.L, E, cfg.window, 0, 13, None, None, 0, None, p0, None, pred)
    _sync()
    p1, _, _ = ost.outputs(1)
    assert np.max(np.abs(from_dev(pred).astype(np.float64) - p1)) <= 1e-6
    p0_ref, P0, _ = ost.outputs(0)
    assert np.max(np.abs(from_dev(pred) - oracle.predict_next(p0_ref, P0))) <= 1e-7


def test_stats_popfetcher_shape():
    cfg = synth.CONFIGS["popfetcher"]
    _run_stats_chain(cfg, cfg.iters, check_every=False)


def test_stats_dsv2_replicas_large_E():
    cfg = synth.CONFIGS["dsv2"].scaled(R=64, window=3)
    _run_stats_chain(cfg, 4)


@pytest.mark.parametrize("E,k,T", [(160, 6, 16384), (181, 8, 700), (182, 8, 700)])
def test_stats_cooccurrence_large_E(E, k, T):
    """Co-occurrence of a 3-layer chain where E*E exceeds 128^2: up to E = 181 a
    block's counts are kept in LDS as packed 16-bit counters (the DeepSeek-V2
    shape at full size: 512 tokens x 36 pairs per block), from E = 182 as packed
    8-bit counters over blocks of 255 tokens; bit-exact against the oracle
    either way."""
    cfg = synth.CONFIGS["dsv2"].scaled(T=T, E=E, k=k, L=3, R=0, window=3, gamma=1.5)
    _run_stats_chain(cfg, 4, check_every=False)


def test_stats_8bit_cooccurrence_counts_duplicates():
    """E = 200 records the co-occurrence in packed 8-bit LDS counters over blocks
    of 255 tokens; tokens that name an expert twice (in this layer or in the
    previous one) count with multiplicity, through global atomics.  Bit-exact
    against the oracle over a 3-layer chain of 3 iterations with such tokens
    in every block."""
    L, E, k, win, T = 3, 200, 3, 2, 700
    state = torch.empty(moe.moe_stats_state_bytes(L, E, win), dtype=torch.uint8, device="cuda")
    moe.moe_stats_init(state, L, E, win)
    ost = oracle.WindowStats(L, E, win)
    outs = {n: torch.empty(sz, dtype=d, device="cuda") for n, sz, d in
            [("counts", E, torch.int32), ("p_seq", E, torch.float32), ("cond", (E, E), torch.float32),
             ("pred", E, torch.float32)]}
    rng = np.random.default_rng(11)
    for it in range(3):
        prev_o, prev_g = None, None
        for layer in range(L):
            lg = (rng.standard_normal((T, E)) - np.log1p(rng.permutation(E))).astype(np.float32)
            idx_o = oracle.route(lg, k)[0].copy()
            for t in (5 + it, 260 + layer, 600):          # one per block of 255 tokens
                idx_o[t, 1] = idx_o[t, 0]
            idx_o[261 + it] = idx_o[261 + it, 2]           # an expert named three times
            idx_g = to_dev(idx_o)
            last = layer + 1 >= L
            moe.moe_stats(state, L, E, win, layer, it, idx_g, prev_g, k, outs["counts"], outs["p_seq"],
                          None if last else outs["cond"], None if last else outs["pred"], 0, None)
            _sync()
            cnt = ost.record(layer, it, idx_o, prev_o)
            assert np.array_equal(from_dev(outs["counts"]), cnt), (it, layer)
            p, P, ph = ost.outputs(layer)
            assert np.max(np.abs(from_dev(outs["p_seq"]) - p)) <= 1e-7
            if not last:
                assert np.max(np.abs(from_dev(outs["cond"]) - P)) <= 1e-7, (it, layer)
                assert np.max(np.abs(from_dev(outs["pred"]) - ph)) <= 1e-6, (it, layer)
            prev_o, prev_g = idx_o, idx_g


def test_stats_maximum_E_and_k():
    """E = 256 experts, top-8, a 3-layer chain: the largest expert count and k the
    library accepts (co-occurrence in packed 8-bit LDS counters)."""
    cfg = synth.CONFIGS["dsv2"].scaled(T=900, E=256, k=8, L=3, R=100, window=4)
    _run_stats_chain(cfg, 5)


# ----------------------------------------------------------------- dispatch
@pytest.mark.parametrize("T,E,k,H,dt,R", [(256, 8, 2, 64, "f32", 4), (1000, 160, 6, 96, "bf16", 0),
                                          (513, 16, 4, 64, "bf16", 16), (1, 8, 2, 8, "bf16", 3),
                                          (300, 32, 2, 40, "f32", 5), (4100, 8, 2, 128, "bf16", 8),
                                          (777, 256, 8, 64, "bf16", 64),
                                          # up to 1024 pairs over up to 64 experts one block does the whole
                                          # dispatch, otherwise three launches: both sides of the boundary
                                          (512, 8, 2, 32, "bf16", 8), (513, 8, 2, 32, "f32", 3),
                                          (256, 64, 4, 16, "bf16", 12), (256, 65, 4, 16, "bf16", 12),
                                          (1024, 16, 1, 16, "f32", 5), (128, 64, 8, 16, "bf16", 20),
                                          (3000, 160, 6, 32, "bf16", 16)])
@pytest.mark.parametrize("plan", [False, True])
def test_dispatch_matches_oracle(T, E, k, H, dt, R, plan):
    """plan: the dispatch plans the replicas itself from the routing's counts
    (replica_budget = R) instead of taking the oracle's plan."""
    lg = _logits(T, E, 7 * T + E, skew=2.0)
    idx_o, _ = oracle.route(lg, k)
    rng = np.random.default_rng(T)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x = synth.f32_to_bf16_bits(x) if dt == "bf16" else x
    reps = oracle.replicas(oracle.histogram(idx_o, E), T, k, R) if R else None
    max_slots = E + R
    if plan:
        d = moe.moe_dispatch(to_dev(x), to_dev(idx_o), E, None, max_slots, replica_budget=R)
    else:
        d = moe.moe_dispatch(to_dev(x), to_dev(idx_o), E, None if reps is None else to_dev(reps), max_slots)
    _sync()
    ref = oracle.dispatch(idx_o, E, reps)
    for key in ("expert_off", "perm_src", "inv_pos"):
        assert np.array_equal(from_dev(d[key]), ref[key]), key
    S = ref["n_slots"]
    assert int(from_dev(d["n_slots"])[0]) == S
    assert np.array_equal(from_dev(d["slot_off"])[:S + 1], ref["slot_off"])
    assert np.all(from_dev(d["slot_off"])[S:] == T * k)
    assert np.array_equal(from_dev(d["slot_expert"])[:S], ref["slot_expert"])
    assert np.array_equal(from_dev(d["x_perm"]), oracle.permute(x, ref["perm_src"]))


def test_dispatch_plan_binding_budget_and_ties():
    """The dispatch's own plan where the budget binds (every copy is handed out)
    and where experts tie on load (ties go to the lower index): the slot table
    equals the oracle's for the oracle's plan of the same counts."""
    T, E, k = 96, 8, 2
    idx = np.zeros((T, k), np.int32)
    idx[:, 0] = np.arange(T) % 4           # experts 0-3 take 24 rows each
    idx[:, 1] = 4 + (np.arange(T) % 2)      # experts 4, 5 take 48 each; 6, 7 none
    for R in (1, 2, 3, 7, 20):
        reps = oracle.replicas(oracle.histogram(idx, E), T, k, R)
        d = moe.moe_dispatch(to_dev(np.zeros((T, 8), np.float32)), to_dev(idx), E, None, E + R, replica_budget=R)
        _sync()
        ref = oracle.dispatch(idx, E, reps)
        S = ref["n_slots"]
        assert int(from_dev(d["n_slots"])[0]) == S, R
        assert np.array_equal(from_dev(d["slot_off"])[:S + 1], ref["slot_off"]), R
        assert np.array_equal(from_dev(d["slot_expert"])[:S], ref["slot_expert"]), R


def test_dispatch_replicas_beyond_budget_are_dropped():
    T, E, k = 64, 4, 2
    idx_o, _ = oracle.route(_logits(T, E, 3), k)
    reps = np.array([5, 1, 7, 2], np.int32)    # 15 copies requested, room for 6
    d = moe.moe_dispatch(to_dev(np.zeros((T, 8), np.float32)), to_dev(idx_o), E, to_dev(reps), E + 6)
    _sync()
    kept = np.array([5, 1, 0, 0], np.int32)     # expert order: 5 + 1 fill the 6 spare slots
    ref = oracle.dispatch(idx_o, E, kept)
    assert int(from_dev(d["n_slots"])[0]) == E + 6
    assert np.array_equal(from_dev(d["slot_off"]), ref["slot_off"])


# ------------------------------------------------------------ whole layer
MINI = {
    "tiny": synth.CONFIGS["tiny"],
    "mixtral-mini": synth.CONFIGS["mixtral"].scaled(T=300, H=256, I=448),
    "dsv2-mini": synth.CONFIGS["dsv2"].scaled(T=200, H=320, I=192),
    "dbrx-mini": synth.CONFIGS["dbrx"].scaled(T=257, H=384, I=640),
    "popf-mini": synth.CONFIGS["popfetcher"].scaled(T=500, H=128, I=256, L=1),
    "max-E-mini": synth.CONFIGS["dsv2"].scaled(T=150, E=256, k=8, H=128, I=192, R=32),
}


def _gpu_layer(cfg, x, lg, wts, R, path="grouped", copy_rows=False):
    wg, wu, wd = (None if w is None else to_dev(w) for w in wts)
    res = moe.moe_layer_forward(to_dev(x), to_dev(lg), cfg.k, wg, wu, wd, cfg.act, R, path=path,
                                copy_rows=copy_rows)
    _sync()
    return res


@pytest.mark.parametrize("name", list(MINI))
@pytest.mark.parametrize("use_reps", [False, True])
@pytest.mark.parametrize("copy_rows", [False, True])
def test_layer_small_elementwise(name, use_reps, copy_rows):
    """copy_rows=False: the FFN gathers its rows from x through perm_src (the
    layer's default); True: the dispatch copies them into x_perm first."""
    cfg = MINI[name]
    R = (cfg.R or 8) if use_reps else 0
    x = synth.hidden0(cfg, 0)
    lg = synth.logits(cfg, 0, 0)
    wts = synth.expert_weights(cfg)
    res = _gpu_layer(cfg, x, lg, wts, R, copy_rows=copy_rows)
    ref = oracle.moe_layer(x, lg, cfg.k, wts, cfg.act, reps_budget=R)
    assert np.array_equal(from_dev(res["idx"]), ref["idx"])
    assert np.array_equal(from_dev(res["perm_src"]), ref["perm_src"])
    if copy_rows:
        assert np.array_equal(from_dev(res["x_perm"]), ref["x_perm"])
    else:
        assert res["x_perm"] is None
    kind = "bf16" if cfg.dtype == "bf16" else "fp32_gemm"
    assert_close(from_dev(res["y_perm"]), ref["y_perm"], kind, "y_perm")
    assert_close(from_dev(res["out"]), ref["out"], kind, "out")


@pytest.mark.parametrize("name", ["mixtral-mini", "dbrx-mini", "popf-mini"])
def test_replication_is_bit_identical(name):
    cfg = MINI[name]
    x = synth.hidden0(cfg, 1)
    lg = synth.logits(cfg, 0, 1)
    wts = synth.expert_weights(cfg)
    a = _gpu_layer(cfg, x, lg, wts, 0)
    ya, oa = from_dev(a["y_perm"]), from_dev(a["out"])
    b = _gpu_layer(cfg, x, lg, wts, cfg.R or 8)
    assert int(from_dev(b["n_slots"])[0]) > cfg.E
    assert np.array_equal(from_dev(b["y_perm"]), ya)
    assert np.array_equal(from_dev(b["out"]), oa)


def test_single_expert_top1_is_dense_ffn():
    cfg = synth.CONFIGS["mixtral"].scaled(T=130, H=128, I=192, E=1, k=1)
    x = synth.hidden0(cfg, 0)
    wts = synth.expert_weights(cfg)
    res = _gpu_layer(cfg, x, np.zeros((cfg.T, 1), np.float32), wts, 0)
    ref = oracle.ffn_rows(x, np.zeros(cfg.T, np.int32), *wts, act="swiglu")
    assert_close(from_dev(res["out"]), ref, "bf16", "out")
    assert np.array_equal(from_dev(res["out"]), from_dev(res["y_perm"]))


# --------------------------------------------- full workload shapes, sampled
def tail_tile_rows(expert_off, tile=256, trailing=4, stride=64):
    """Rows chosen where the grouped GEMM's tiles are partial or re-listed: the
    first and last row of every expert's last `tile`-row tile (a range of at most
    64 rows is one 64-row tile), and one row per `stride` rows (plus the last) of
    the table's last `trailing` tiles, which the launch may run again as 64-row
    tiles.  Consecutive replica slots of an expert are tiled as one range, so the
    expert ranges are the tile ranges."""
    off = np.asarray(expert_off, np.int64)
    rows, tiles = set(), []
    for e in range(len(off) - 1):
        a, b = int(off[e]), int(off[e + 1])
        if b > a:
            rows.update((b - 1, a + (b - 1 - a) // tile * tile))
            tiles.extend((t0, min(t0 + tile, b)) for t0 in range(a, b, tile))
    for t0, t1 in tiles[-trailing:]:
        rows.update(range(t0, t1, stride))
        rows.add(t1 - 1)
    return np.array(sorted(rows), np.int64)


def _sampled_layer_check(cfg, R, n_sample=12, seed=0, copy_rows=False):
    x = synth.hidden0(cfg, 0)
    lg = synth.logits(cfg, 0, 0)
    wts = synth.expert_weights(cfg, threads=16)
    res = _gpu_layer(cfg, x, lg, wts, R, copy_rows=copy_rows)
    idx_o, w_o = oracle.route(lg, cfg.k)
    assert np.array_equal(from_dev(res["idx"]), idx_o)
    reps = oracle.replicas(oracle.histogram(idx_o, cfg.E), cfg.T, cfg.k, R) if R else None
    d = oracle.dispatch(idx_o, cfg.E, reps)
    for key in ("expert_off", "perm_src", "inv_pos"):
        assert np.array_equal(from_dev(res[key]), d[key]), key
    S = d["n_slots"]
    assert np.array_equal(from_dev(res["slot_off"])[:S + 1], d["slot_off"])
    kind = "bf16" if cfg.dtype == "bf16" else "fp32_gemm"
    # y_perm rows in every expert's partial last tile and in the trailing tiles
    rows = tail_tile_rows(d["expert_off"])
    row_expert = np.repeat(np.arange(cfg.E, dtype=np.int32), np.diff(d["expert_off"]))
    y_rows = oracle.ffn_rows(x[d["perm_src"][rows]], row_expert[rows], *wts, act=cfg.act)
    assert_close(from_dev(res["y_perm"])[rows], y_rows, kind, f"y_perm rows of the tail tiles ({rows.size})")
    # whole tokens (all k slots, combine): seeded sample
    sample = np.random.default_rng(seed).choice(cfg.T, size=n_sample, replace=False)
    y_ref, out_ref = oracle.token_forward(x[sample], idx_o[sample], w_o[sample], wts, cfg.act)
    y_gpu = from_dev(res["y_perm"])[d["inv_pos"][sample].ravel()].reshape(y_ref.shape)
    assert_close(y_gpu, y_ref, kind, "sampled y_perm rows")
    assert_close(from_dev(res["out"])[sample], out_ref, kind, "sampled out rows")
    if copy_rows:
        x_perm = from_dev(res["x_perm"])
        rows = np.random.default_rng(seed + 1).choice(cfg.T * cfg.k, size=256, replace=False)
        assert np.array_equal(x_perm[rows], x[d["perm_src"][rows]])
    return res


@pytest.mark.parametrize("R", [0, 8])
def test_mixtral_full_size_sampled(R):
    _sampled_layer_check(synth.CONFIGS["mixtral"], R)


@pytest.mark.parametrize("T", synth.DSV2_T_SWEEP)
def test_dsv2_full_size_sampled(T):
    _sampled_layer_check(synth.CONFIGS["dsv2"].with_T(T), 0, n_sample=6)


def test_dbrx_full_size_replication_equivalence():
    cfg = synth.CONFIGS["dbrx"]
    res = _sampled_layer_check(cfg, cfg.R, n_sample=6)
    y_rep, out_rep = from_dev(res["y_perm"]), from_dev(res["out"])
    del res
    x = synth.hidden0(cfg, 0)
    lg = synth.logits(cfg, 0, 0)
    wts = synth.expert_weights(cfg, threads=16)
    plain = _gpu_layer(cfg, x, lg, wts, 0)
    assert np.array_equal(from_dev(plain["y_perm"]), y_rep)
    assert np.array_equal(from_dev(plain["out"]), out_rep)


def test_popfetcher_full_chain_sampled():
    """12 chained fp32 GELU layers at T=16384: routing bit-exact at every layer,
    and the final hidden states of sampled tokens against the oracle's per-token
    chain (a token's trajectory depends only on its own row)."""
    cfg = synth.CONFIGS["popfetcher"]
    sample = np.random.default_rng(5).choice(cfg.T, size=8, replace=False)
    x = synth.hidden0(cfg, 0)
    xg = to_dev(x)
    xs = x[sample]
    prev = None
    bufs = {}
    for layer in range(cfg.L):
        wts = synth.expert_weights(cfg, layer=layer, threads=16)
        lg = synth.logits(cfg, layer, 0, None if prev is None else prev[:, 0])
        wg, _, wd = (None if w is None else to_dev(w) for w in wts)
        res = moe.moe_layer_forward(xg, to_dev(lg), cfg.k, wg, None, wd, cfg.act, 0, bufs=bufs)
        _sync()
        idx_o, w_o = oracle.route(lg, cfg.k)
        assert np.array_equal(from_dev(res["idx"]), idx_o), layer
        _, xs = oracle.token_forward(xs, idx_o[sample], w_o[sample], wts, cfg.act)
        xg = res["out"].clone()
        prev = idx_o
    assert_close(from_dev(xg)[sample], xs, "fp32_gemm", "layer-12 hidden states (sampled)")


# ------------------------------------------------ grouped vs dense vs auto
@pytest.mark.parametrize("name", ["tiny", "mixtral-mini", "dsv2-mini", "popf-mini"])
def test_gemm_paths_are_bit_identical(name):
    """The dense padded batch (64-row tiles), the grouped 64-row and 256-row tiles
    compute every row with the same K order: identical bits."""
    cfg = MINI[name]
    x = synth.hidden0(cfg, 2)
    lg = synth.logits(cfg, 0, 2)
    wts = synth.expert_weights(cfg)
    ref = oracle.moe_layer(x, lg, cfg.k, wts, cfg.act)
    outs = {}
    for path in ("grouped", "dense", "grouped_small", "auto"):
        res = _gpu_layer(cfg, x, lg, wts, 0, path=path)
        outs[path] = (from_dev(res["y_perm"]), from_dev(res["out"]))
    for path in ("dense", "grouped_small", "auto"):
        assert np.array_equal(outs[path][0], outs["grouped"][0]), path
        assert np.array_equal(outs[path][1], outs["grouped"][1]), path
    kind = "bf16" if cfg.dtype == "bf16" else "fp32_gemm"
    assert_close(outs["dense"][1], ref["out"], kind, "dense out")


@pytest.mark.parametrize("H,I", [(192, 320), (448, 128), (64, 384)])
def test_direct_to_lds_tiles_partial_columns_odd_k(H, I):
    """The bf16 256-row tiles (operands fetched straight into LDS, the K loop
    unrolled six steps at a time) on shapes with partial column tiles and K-step
    counts 1, 2, 3, 5, 6 and 7 (every remainder of the unrolled loop but 4, which
    the Mixtral shape covers): e.g. I = 320 leaves the last gate/up tile 64 of 128
    columns and H = 192 the down tile 192 of 256.  Two experts, top-2: 86 row
    tiles of 256, so the grid keeps most of them.  Sampled tokens match the oracle
    and the whole output equals the all-64-row path bit for bit."""
    cfg = synth.CONFIGS["mixtral"].scaled(T=11008, E=2, H=H, I=I)
    res = _sampled_layer_check(cfg, 0, n_sample=16)
    y_g, out_g = res["y_perm"], res["out"]
    x = synth.hidden0(cfg, 0)
    lg = synth.logits(cfg, 0, 0)
    wts = synth.expert_weights(cfg, threads=16)
    small = _gpu_layer(cfg, x, lg, wts, 0, path="grouped_small")
    assert torch.equal(small["y_perm"], y_g)
    assert torch.equal(small["out"], out_g)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M", [900, 30000])
def test_expert_ffn_gathers_rows_like_a_copy(M, dtype):
    """moe_expert_ffn with a row map (row_src) over a token matrix: repeated
    rows, every row order, and map entries outside [0, n_src) (read as zero
    rows).  Every path gives the bits of the FFN of the same rows copied out on
    the host, and the rows match the oracle's FFN."""
    n_src = M // 3 + 7
    cfg = synth.CONFIGS["mixtral"].scaled(T=n_src, E=3, H=128, I=192, dtype=dtype)
    x = synth.hidden0(cfg, 5)
    wts = synth.expert_weights(cfg)
    rng = np.random.default_rng(M)
    row_src = rng.integers(0, n_src, size=M).astype(np.int32)
    row_src[rng.choice(M, size=5, replace=False)] = np.array([-1, n_src, n_src + 100, -7, 2 ** 30], np.int32)
    gathered = np.where((row_src >= 0)[:, None] & (row_src < n_src)[:, None],
                        x[np.clip(row_src, 0, n_src - 1)], np.zeros_like(x[:1]))
    cuts = [0, M // 4, M // 4, (3 * M) // 5, M]
    experts = [1, 0, 2, 1]
    max_slots = 6
    slot_off = np.full(max_slots + 1, M, np.int32)
    slot_off[:len(cuts)] = cuts
    slot_expert = np.zeros(max_slots, np.int32)
    slot_expert[:len(experts)] = experts
    n_slots = np.array([len(experts)], np.int32)
    wg, wu, wd = (to_dev(w) for w in wts)
    so, se, ns = to_dev(slot_off), to_dev(slot_expert), to_dev(n_slots)
    xd, rs, gd = to_dev(x), to_dev(row_src), to_dev(gathered)
    ref = oracle.ffn_rows(gathered, np.repeat(np.array(experts, np.int32), np.diff(cuts)), *wts, act="swiglu")
    for path in ("grouped", "grouped_small", "dense", "auto"):
        y_gather = moe.moe_expert_ffn(xd, so, se, ns, wg, wu, wd, act="swiglu", path=path, row_src=rs)
        y_copy = moe.moe_expert_ffn(gd, so, se, ns, wg, wu, wd, act="swiglu", path=path)
        _sync()
        assert torch.equal(y_gather, y_copy), path
        if path == "grouped":
            assert_close(from_dev(y_gather), ref, "bf16" if dtype == "bf16" else "fp32_gemm", "y_perm")


def test_mixtral_full_size_gather_equals_copy():
    """The full Mixtral-shaped layer (R = 8): the gathering FFN (the layer's
    default) and the copying dispatch + FFN give the same bits."""
    cfg = synth.CONFIGS["mixtral"]
    x = synth.hidden0(cfg, 0)
    lg = synth.logits(cfg, 0, 0)
    wts = synth.expert_weights(cfg, threads=16)
    a = _gpu_layer(cfg, x, lg, wts, 8)
    out_a, y_a = a["out"].clone(), a["y_perm"].clone()
    del a
    b = _gpu_layer(cfg, x, lg, wts, 8, copy_rows=True)
    assert torch.equal(b["y_perm"], y_a)
    assert torch.equal(b["out"], out_a)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("M", [900, 30000])
def test_expert_ffn_hand_made_slot_table(M, dtype):
    """moe_expert_ffn on a slot table dispatch never produces: expert 0's rows in
    two non-adjacent slots, two adjacent slots of expert 1 (tiled as one range),
    an empty slot and unused slot capacity.  Every row matches the oracle's FFN of
    its slot's expert, and the four paths give the same bits."""
    cfg = synth.CONFIGS["mixtral"].scaled(T=M, E=3, H=128, I=192, dtype=dtype)
    x = synth.hidden0(cfg, 3)
    wts = synth.expert_weights(cfg)
    cuts = [0, M // 9, M // 9, M // 3, (2 * M) // 3, (2 * M) // 3 + 1, M]
    experts = [0, 2, 1, 1, 0, 2]
    max_slots = 8
    slot_off = np.full(max_slots + 1, M, np.int32)
    slot_off[:len(cuts)] = cuts
    slot_expert = np.zeros(max_slots, np.int32)
    slot_expert[:len(experts)] = experts
    n_slots = np.array([len(experts)], np.int32)
    ref = oracle.ffn_rows(x, np.repeat(np.array(experts, np.int32), np.diff(cuts)), *wts, act="swiglu")
    wg, wu, wd = (to_dev(w) for w in wts)
    xd, so, se, ns = to_dev(x), to_dev(slot_off), to_dev(slot_expert), to_dev(n_slots)
    outs = {}
    for path in ("grouped", "grouped_small", "dense", "auto"):
        y = moe.moe_expert_ffn(xd, so, se, ns, wg, wu, wd, act="swiglu", path=path)
        _sync()
        outs[path] = from_dev(y)
    assert_close(outs["grouped"], ref, "bf16" if dtype == "bf16" else "fp32_gemm", "y_perm")
    for path in ("grouped_small", "dense", "auto"):
        assert np.array_equal(outs[path], outs["grouped"]), path


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_grouped_128_row_tail_tiles(dtype):
    """In a wide gate/up GEMM (I = 4096: 32 column tiles), ranges whose last
    256-row tile holds at most 128 rows run it as a 128-row tile (bf16 SwiGLU;
    the down GEMM keeps 256-row tiles): ranges of 64 (short), 65, 100, 128, 129,
    256, 257 (a 1-row tail), 300, 384, 385 and 641 rows, with replicas of one
    expert as adjacent slots.  Every row matches the oracle and all paths give
    the same bits (fp32 has no 128-row tiles: the same table runs on 256-row
    tiles)."""
    sizes = [64, 65, 100, 128, 129, 256, 257, 300, 384, 385, 641]
    experts = list(range(len(sizes)))
    experts[-1] = experts[-2] = 9          # 385 + 641 rows of one expert (two replica slots)
    E = 10
    cuts = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(cuts[-1])
    cfg = synth.CONFIGS["mixtral"].scaled(T=M, E=E, H=128, I=4096, dtype=dtype)
    x = synth.hidden0(cfg, 5)
    wts = synth.expert_weights(cfg)
    max_slots = len(sizes) + 2
    slot_off = np.full(max_slots + 1, M, np.int32)
    slot_off[:len(cuts)] = cuts
    slot_expert = np.zeros(max_slots, np.int32)
    slot_expert[:len(experts)] = experts
    ref = oracle.ffn_rows(x, np.repeat(np.array(experts, np.int32), sizes), *wts, act="swiglu")
    wg, wu, wd = (to_dev(w) for w in wts)
    args = (to_dev(x), to_dev(slot_off), to_dev(slot_expert), to_dev(np.array([len(sizes)], np.int32)))
    outs = {}
    for path in ("grouped", "grouped_small", "dense", "auto"):
        outs[path] = from_dev(moe.moe_expert_ffn(*args, wg, wu, wd, act="swiglu", path=path))
    _sync()
    assert_close(outs["grouped"], ref, "bf16" if dtype == "bf16" else "fp32_gemm", "y_perm")
    for path in ("grouped_small", "dense", "auto"):
        assert np.array_equal(outs[path], outs["grouped"]), path


@pytest.mark.parametrize("dtype,n,max_rows", [("bf16", 300, 520), ("f32", 300, 520), ("bf16", 1100, 100)])
def test_grouped_remainder_tiles_and_last_round(dtype, n, max_rows):
    """The 256-row grouped tiling on 300 slots (more than one 256-slot chunk of
    the tile-table scan) over 40 experts, slot sizes 0..519 with planted 1, 64,
    65, 255, 256 and 257: the 41 ranges of at most 64 rows run as 64-row tiles
    in the same launch, and both GEMMs (two and one column tiles) list trailing
    row tiles again as 64-row tiles to fill the launch's last round.  With 1100
    slots (sizes 0..99) the tile-table kernel reads the slot table from global
    memory instead of LDS.  Every row matches the oracle's FFN of its slot's
    expert; all paths give the same bits."""
    rng = np.random.default_rng(11)
    sizes = rng.integers(0, max_rows, n)
    sizes[::17] = 0
    sizes[[5, 6, 7, 8, 9, 10]] = [64, 65, 256, 257, 1, 255]
    experts = rng.integers(0, 40, n).astype(np.int32)
    M = int(sizes.sum())
    cfg = synth.CONFIGS["mixtral"].scaled(T=M, E=40, H=128, I=192, dtype=dtype)
    x = synth.hidden0(cfg, 5)
    wts = synth.expert_weights(cfg)
    max_slots = n + 20
    slot_off = np.full(max_slots + 1, M, np.int32)
    slot_off[:n + 1] = np.concatenate([[0], np.cumsum(sizes)])
    slot_expert = np.zeros(max_slots, np.int32)
    slot_expert[:n] = experts
    ref = oracle.ffn_rows(x, np.repeat(experts, sizes), *wts, act="swiglu")
    wg, wu, wd = (to_dev(w) for w in wts)
    xd, so, se, ns = to_dev(x), to_dev(slot_off), to_dev(slot_expert), to_dev(np.array([n], np.int32))
    outs = {}
    for path in ("grouped", "grouped_small", "dense", "auto"):
        y = moe.moe_expert_ffn(xd, so, se, ns, wg, wu, wd, act="swiglu", path=path)
        _sync()
        outs[path] = from_dev(y)
    assert_close(outs["grouped"], ref, "bf16" if dtype == "bf16" else "fp32_gemm", "y_perm")
    for path in ("grouped_small", "dense", "auto"):
        assert np.array_equal(outs[path], outs["grouped"]), path


def test_tail_retiling_full_size_mixtral():
    """Mixtral shape: the down GEMM's 256-row tiles fill 4.25 rounds of the 256
    CUs, so the grouped path lists the trailing row tiles again as 64-row tiles
    that run in the same launch.  Every row keeps its K order: the grouped output
    equals the all-64-row path bit for bit, with and without replica slots."""
    cfg = synth.CONFIGS["mixtral"]
    x = synth.hidden0(cfg, 0)
    lg = synth.logits(cfg, 0, 0)
    wts = synth.expert_weights(cfg, threads=16)
    wg, wu, wd = (to_dev(w) for w in wts)
    xd, lgd = to_dev(x), to_dev(lg)
    for R in (0, 8):
        outs = {}
        for path in ("grouped", "grouped_small"):
            res = moe.moe_layer_forward(xd, lgd, cfg.k, wg, wu, wd, cfg.act, R, path=path)
            _sync()
            outs[path] = (res["y_perm"], res["out"])
        assert torch.equal(outs["grouped"][0], outs["grouped_small"][0]), R
        assert torch.equal(outs["grouped"][1], outs["grouped_small"][1]), R


def test_dense_path_full_size_dsv2_small_batch():
    """DeepSeek-V2 shape at T=1024: many small and some empty experts, where the
    64-row tilings win; the dense, grouped-small and auto paths must equal the
    grouped path bit for bit."""
    cfg = synth.CONFIGS["dsv2"].with_T(1024)
    x = synth.hidden0(cfg, 0)
    lg = synth.logits(cfg, 0, 0)
    wts = synth.expert_weights(cfg, threads=16)
    g = _gpu_layer(cfg, x, lg, wts, 0, path="grouped")
    yg, og = from_dev(g["y_perm"]), from_dev(g["out"])
    for path in ("dense", "grouped_small", "auto"):
        d = _gpu_layer(cfg, x, lg, wts, 0, path=path)
        assert np.array_equal(from_dev(d["y_perm"]), yg), path
        assert np.array_equal(from_dev(d["out"]), og), path
