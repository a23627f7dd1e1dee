"""Device-check mode: each hot-path call ORs a MOE_CHECK_* bit into the caller's
check word for the invalid input it meets, skips that input (no fault, indices
stay in range) and moe_check_device_error reports the bits; valid inputs flag
nothing.  Every case here is memory-safe by the kernels' own bounds: invalid
entries are skipped, never dereferenced."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_top_amd as moe
import oracle
import synth
from _util import from_dev, to_dev

pytestmark = pytest.mark.gpu
B = moe.CHECK_BITS


def _word():
    return moe.new_check_word()


def _bits(word):
    try:
        return moe.moe_check_device_error(word)
    except moe.MoEError as e:
        assert e.status == -5, e
        bits = int(word.item())
        assert bits != 0
        return bits


def _logits(T, E, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((T, E)) - np.log1p(rng.permutation(E))).astype(np.float32)


def test_valid_layer_flags_nothing():
    cfg = synth.CONFIGS["mixtral"].scaled(T=300, H=256, I=448)
    x, lg = synth.hidden0(cfg, 0), synth.logits(cfg, 0, 0)
    wg, wu, wd = (to_dev(w) for w in synth.expert_weights(cfg))
    word = _word()
    state = torch.empty(moe.moe_stats_state_bytes(2, cfg.E, 4), dtype=torch.uint8, device="cuda")
    moe.moe_stats_init(state, 2, cfg.E, 4)
    prev, _ = moe.moe_route(to_dev(_logits(cfg.T, cfg.E, 1)), cfg.k)
    res = moe.moe_layer_forward(to_dev(x), to_dev(lg), cfg.k, wg, wu, wd, "swiglu", 8, stats_state=state,
                                stats_dims=(2, cfg.E, 4), layer=1, it=0, prev_topk_idx=prev, check=word)
    assert moe.moe_check_device_error(word) == 0
    ref = oracle.moe_layer(x, lg, cfg.k, synth.expert_weights(cfg), "swiglu", reps_budget=8)
    assert np.array_equal(from_dev(res["inv_pos"]), ref["inv_pos"])


def test_route_flags_non_finite_logits():
    T, E, k = 200, 16, 4
    lg = _logits(T, E, 2)
    word = _word()
    moe.moe_route(to_dev(lg), k, check=word)
    assert moe.moe_check_device_error(word) == 0
    for bad in (np.nan, np.inf, -np.inf):
        bl = lg.copy()
        bl[37, 5] = bad
        word = _word()
        idx, _ = moe.moe_route(to_dev(bl), k, check=word)
        assert _bits(word) == B["logits"], bad
        got = from_dev(idx)
        assert got.min() >= 0 and got.max() < E
        assert all(len(set(r)) == k for r in got.tolist())          # k distinct experts still
        assert np.array_equal(np.delete(got, 37, axis=0), np.delete(oracle.route(lg, k)[0], 37, axis=0))


def test_stats_flags_out_of_range_and_duplicate_indices():
    T, E, k, L, win = 300, 8, 2, 2, 3
    idx = oracle.route(_logits(T, E, 3), k)[0]
    prev = oracle.route(_logits(T, E, 4), k)[0]
    state = torch.empty(moe.moe_stats_state_bytes(L, E, win), dtype=torch.uint8, device="cuda")
    moe.moe_stats_init(state, L, E, win)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    word = _word()
    moe.moe_stats(state, L, E, win, 1, 0, to_dev(idx), to_dev(prev), k, counts, check=word)
    assert moe.moe_check_device_error(word) == 0
    bad = idx.copy()
    bad[3] = [-1, E + 3]          # out of range: skipped
    bad[9] = [5, 5]               # a duplicate: counted twice
    word = _word()
    moe.moe_stats(state, L, E, win, 1, 1, to_dev(bad), to_dev(prev), k, counts, check=word)
    assert _bits(word) == B["index"] | B["duplicate"]
    valid = bad[(bad >= 0) & (bad < E)]
    assert np.array_equal(from_dev(counts), np.bincount(valid, minlength=E))


# T*k up to 1024 (at most 64 experts) runs the one-block dispatch, above it the three-launch path
@pytest.mark.parametrize("T", [200, 4400])
def test_dispatch_duplicate_indices_match_the_oracle(T):
    """A token naming one expert twice gets two rows in slot order (the stable
    order of the flattened pairs, as the oracle defines it), and is flagged."""
    E, k, H = 16, 4, 64
    idx = oracle.route(_logits(T, E, 5), k)[0]
    idx[0] = [3, 3, 3, 1]
    idx[T // 2] = [7, 2, 7, 2]
    x = synth.f32_to_bf16_bits(np.random.default_rng(0).standard_normal((T, H)).astype(np.float32))
    word = _word()
    d = moe.moe_dispatch(to_dev(x), to_dev(idx), E, None, E, check=word)
    assert _bits(word) == B["duplicate"]
    ref = oracle.dispatch(idx, E)
    for key in ("expert_off", "perm_src", "inv_pos", "slot_off"):
        assert np.array_equal(from_dev(d[key]), ref[key]), key
    assert np.array_equal(from_dev(d["x_perm"]), oracle.permute(x, ref["perm_src"]))


@pytest.mark.parametrize("T", [300, 9000])
def test_dispatch_skips_out_of_range_indices(T):
    E, k, H = 8, 2, 32
    idx = oracle.route(_logits(T, E, 6), k)[0]
    idx[10, 1] = E
    idx[T - 100, 0] = -7
    x = np.random.default_rng(1).standard_normal((T, H)).astype(np.float32)
    word = _word()
    d = moe.moe_dispatch(to_dev(x), to_dev(idx), E, None, E, check=word)
    assert _bits(word) == B["index"]
    inv = from_dev(d["inv_pos"])
    assert inv[10, 1] == -1 and inv[T - 100, 0] == -1
    # the valid pairs: stable order by expert, then pair index
    flat = idx.ravel()
    ok = np.flatnonzero((flat >= 0) & (flat < E))
    order = ok[np.argsort(flat[ok], kind="stable")]
    n = order.size
    assert np.array_equal(from_dev(d["expert_off"]), np.concatenate([[0], np.cumsum(np.bincount(flat[ok], minlength=E))]))
    assert np.array_equal(from_dev(d["perm_src"])[:n], order // k)
    assert np.array_equal(inv.ravel()[order], np.arange(n))
    assert np.array_equal(from_dev(d["x_perm"])[:n], x[order // k])


@pytest.mark.parametrize("T", [256, 8500])
def test_dispatch_flags_counts_and_replica_budget(T):
    E, k = 8, 2
    idx = oracle.route(_logits(T, E, 7), k)[0]
    n = np.bincount(idx.ravel(), minlength=E).astype(np.int32)
    x = to_dev(np.zeros((T, 8), np.float32))
    word = _word()
    moe.moe_dispatch(x, to_dev(idx), E, None, E, counts=to_dev(n), check=word)
    assert moe.moe_check_device_error(word) == 0
    wrong = n.copy()
    wrong[2] += 1
    word = _word()
    moe.moe_dispatch(x, to_dev(idx), E, None, E, counts=to_dev(wrong), check=word)
    assert _bits(word) == B["counts"]
    for reps, slots in ((np.array([0, 5, 0, 0, 3, 0, 0, 0], np.int32), E + 4),   # 8 copies, room for 4
                        (np.array([0, -1, 0, 0, 0, 0, 0, 0], np.int32), E + 4)):  # negative
        word = _word()
        d = moe.moe_dispatch(x, to_dev(idx), E, to_dev(reps), slots, check=word)
        assert _bits(word) == B["replicas"]
        kept = np.maximum(reps, 0)
        room = slots - E
        kept = np.array([max(0, min(r, room - kept[:e].sum())) for e, r in enumerate(kept)], np.int32)
        ref = oracle.dispatch(idx, E, kept)
        S = ref["n_slots"]
        assert np.array_equal(from_dev(d["slot_off"])[:S + 1], ref["slot_off"])


def test_ffn_flags_an_invalid_slot_table():
    cfg = synth.CONFIGS["mixtral"].scaled(T=64, H=128, I=192)
    E, M, H = cfg.E, cfg.T * cfg.k, cfg.H
    wg, wu, wd = (to_dev(w) for w in synth.expert_weights(cfg))
    x = to_dev(synth.f32_to_bf16_bits(np.random.default_rng(2).standard_normal((M, H)).astype(np.float32)))
    good_off = np.array([0, 10, 10, 40, 64, 64, 90, 100, M], np.int32)
    good_se = np.arange(E, dtype=np.int32)
    ns = to_dev(np.array([E], np.int32))
    word = _word()
    y0 = moe.moe_expert_ffn(x, to_dev(good_off), to_dev(good_se), ns, wg, wu, wd, check=word)
    assert moe.moe_check_device_error(word) == 0
    for off, se, n in ((good_off, np.where(good_se == 3, E + 2, good_se).astype(np.int32), E),  # expert out of range
                       (np.array([0, 10, 5, 40, 64, 64, 90, 100, M], np.int32), good_se, E),     # not ascending
                       (np.array([0, 10, 10, 40, 64, 64, 90, 100, M + 9], np.int32), good_se, E),  # past M
                       (good_off, good_se, E + 1)):                                             # n_slots > max
        word = _word()
        y = moe.moe_expert_ffn(x, to_dev(off), to_dev(se), to_dev(np.array([n], np.int32)), wg, wu, wd, check=word)
        assert _bits(word) == B["slots"]
    # rows of valid slots are still computed as before (first slot untouched)
    assert torch.equal(y[:10], y0[:10])


def test_combine_flags_rows_out_of_range():
    T, k, H = 100, 2, 64
    M = T * k
    y = to_dev(np.random.default_rng(3).standard_normal((M, H)).astype(np.float32))
    inv = np.arange(M, dtype=np.int32).reshape(T, k)
    w = to_dev(np.full((T, k), 0.5, np.float32))
    word = _word()
    ref = moe.moe_combine(y, to_dev(inv), w, check=word)
    assert moe.moe_check_device_error(word) == 0
    bad = inv.copy()
    bad[4, 1] = -1
    bad[50, 0] = M + 5
    word = _word()
    out = moe.moe_combine(y, to_dev(bad), w, check=word)
    assert _bits(word) == B["rows"]
    keep = np.setdiff1d(np.arange(T), [4, 50])
    assert torch.equal(out[keep], ref[keep])
    yy = from_dev(y)
    assert np.allclose(from_dev(out)[4], 0.5 * yy[inv[4, 0]])


def test_check_word_accumulates_until_cleared():
    T, E, k = 64, 8, 2
    lg = _logits(T, E, 8)
    lg[0, 0] = np.nan
    word = _word()
    moe.moe_route(to_dev(lg), k, check=word)
    idx = oracle.route(_logits(T, E, 9), k)[0]
    idx[1] = [4, 4]
    moe.moe_dispatch(to_dev(np.zeros((T, 8), np.float32)), to_dev(idx), E, None, E, check=word)
    assert _bits(word) == B["logits"] | B["duplicate"]
    word.zero_()
    assert moe.moe_check_device_error(word) == 0


def test_binding_rejects_mismatched_buffers_before_any_launch():
    """Outputs and workspaces handed to the binding are checked against the sizes
    the kernels will write before anything is enqueued; cached layer buffers
    are reallocated when T, k or the replica budget change."""
    T, E, k, H = 100, 8, 2, 64
    lg = to_dev(_logits(T, E, 10))
    small = torch.full((T // 2, k), -5, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError):
        moe.moe_route(lg, k, topk_idx=small)
    torch.cuda.synchronize()
    assert torch.all(small == -5)
    x = to_dev(np.random.default_rng(4).standard_normal((T, H)).astype(np.float32))
    idx, _ = moe.moe_route(lg, k)
    d = moe.moe_dispatch(x, idx, E, None, E)
    x2 = to_dev(np.random.default_rng(5).standard_normal((2 * T, H)).astype(np.float32))
    idx2, _ = moe.moe_route(to_dev(_logits(2 * T, E, 11)), k)
    before = d["x_perm"].clone()
    with pytest.raises(ValueError):
        moe.moe_dispatch(x2, idx2, E, None, E, out=d)              # buffers sized for T rows
    with pytest.raises(ValueError):
        moe.moe_dispatch(x2, idx2, E, None, E, workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(d["x_perm"], before)
    # one bufs dict across a change of T and of the replica budget
    cfg = synth.CONFIGS["mixtral"].scaled(T=100, H=128, I=192)
    wts = synth.expert_weights(cfg)
    wg, wu, wd = (to_dev(w) for w in wts)
    bufs = {}
    for T_, R_ in ((100, 0), (260, 8), (90, 3)):
        c = cfg.with_T(T_)
        xx, ll = synth.hidden0(c, 0), synth.logits(c, 0, 0)
        got = moe.moe_layer_forward(to_dev(xx), to_dev(ll), c.k, wg, wu, wd, "swiglu", R_, bufs=bufs)
        fresh = moe.moe_layer_forward(to_dev(xx), to_dev(ll), c.k, wg, wu, wd, "swiglu", R_)
        assert torch.equal(got["out"], fresh["out"]) and got["slot_off"].numel() == c.E + R_ + 1
    # pipelined chunks: per-chunk buffers keyed on each chunk's own size
    c = cfg.with_T(9)
    xx, ll = to_dev(synth.hidden0(c, 0)), to_dev(synth.logits(c, 0, 0))
    ref = moe.moe_layer_forward(xx, ll, c.k, wg, wu, wd, "swiglu", 0)["out"]
    pb = {}
    for n in (4, 3, 2):
        res = moe.moe_layer_forward_pipelined(xx, ll, c.k, wg, wu, wd, "swiglu", n, bufs=pb)
        torch.cuda.synchronize()
        assert torch.equal(res["out"], ref), n
