"""Pins for the CPU oracle: each check compares it with something other than
itself -- a textbook/library routine, a closed form, an invariant the pages fix,
brute force on tiny inputs, or a hand-derived worked example (tests/golden)."""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def _rand_logits(T, E, seed):
    return np.random.default_rng(seed).standard_normal((T, E)).astype(np.float32)


# ---------------------------------------------------------------- routing
@pytest.mark.parametrize("E,k", [(8, 2), (16, 4), (160, 6), (32, 2), (5, 5)])
def test_route_matches_stable_argsort(E, k):
    for logits in (_rand_logits(300, E, E * 10 + k), synth.tie_logits(300, E)):
        idx, _ = oracle.route(logits, k)
        ref = np.argsort(-logits, axis=1, kind="stable")[:, :k]
        assert np.array_equal(idx, ref)


def test_route_bruteforce_subsets():
    """Exactly one k-subset S satisfies: every e in S beats every e' outside (higher
    logit, or equal logit and lower index); it must be the oracle's set."""
    rng = np.random.default_rng(3)
    for trial in range(200):
        E = int(rng.integers(2, 7))
        k = int(rng.integers(1, E + 1))
        row = (rng.integers(-2, 3, size=E) * 0.5).astype(np.float32)
        beats = lambda a, b: row[a] > row[b] or (row[a] == row[b] and a < b)
        winners = [S for S in itertools.combinations(range(E), k)
                   if all(beats(a, b) for a in S for b in range(E) if b not in S)]
        assert len(winners) == 1
        idx, _ = oracle.route(row[None, :], k)
        assert set(idx[0].tolist()) == set(winners[0])
        # slot order: descending logit, ties by index
        assert all(beats(idx[0][i], idx[0][i + 1]) for i in range(k - 1))


def test_route_k2_closed_form():
    logits = _rand_logits(1000, 8, 11)
    idx, w = oracle.route(logits, 2)
    l0 = logits[np.arange(1000), idx[:, 0]].astype(np.float64)
    l1 = logits[np.arange(1000), idx[:, 1]].astype(np.float64)
    w0 = 1.0 / (1.0 + np.exp(l1 - l0))
    assert np.all(np.abs(w[:, 0] - w0) <= 2.0 ** -24 * 2)
    assert np.all(np.abs(w[:, 1] - (1.0 - w0)) <= 2.0 ** -24 * 2)


def test_route_k_equals_E_is_full_softmax():
    logits = _rand_logits(200, 6, 12)
    idx, w = oracle.route(logits, 6)
    sm = torch.softmax(torch.from_numpy(logits).double(), dim=1).numpy()
    ref = np.take_along_axis(sm, idx.astype(np.int64), axis=1)
    assert np.max(np.abs(w - ref)) <= 2.0 ** -23


def test_route_weights_sum_to_one():
    for E, k in [(8, 2), (160, 6), (16, 4)]:
        _, w = oracle.route(_rand_logits(500, E, E), k)
        assert np.max(np.abs(w.astype(np.float64).sum(1) - 1.0)) <= 2.0 ** -22 * k


def test_route_golden():
    for case in GOLD["route"]:
        idx, w = oracle.route(np.array(case["logits"], np.float32), case["k"])
        assert idx.tolist() == case["idx"], case["cite"]
        assert np.array_equal(w, np.array(case["w"], np.float32)), case["cite"]


# ------------------------------------------------------------- statistics
def test_histogram_counts():
    logits = _rand_logits(777, 16, 5)
    idx, _ = oracle.route(logits, 4)
    n = oracle.histogram(idx, 16)
    assert n.sum() == 777 * 4
    assert np.array_equal(n, np.bincount(idx.ravel(), minlength=16))


def _onehot_counts(idx, E):
    A = np.zeros((idx.shape[0], E), np.int64)
    for i in range(idx.shape[1]):
        np.add.at(A, (np.arange(idx.shape[0]), idx[:, i]), 1)
    return A


@pytest.mark.parametrize("E,k", [(8, 2), (32, 2), (16, 4), (6, 1)])
def test_cooccurrence_matrix_identities(E, k):
    rng = np.random.default_rng(E + k)
    prev, _ = oracle.route(rng.standard_normal((400, E)).astype(np.float32), k)
    nxt, _ = oracle.route(rng.standard_normal((400, E)).astype(np.float32), k)
    C = oracle.cooccurrence(prev, nxt, E)
    # textbook: C = A_prev^T A_next with per-token expert-count rows
    assert np.array_equal(C, _onehot_counts(prev, E).T @ _onehot_counts(nxt, E))
    assert np.array_equal(C.sum(1), k * np.bincount(prev.ravel(), minlength=E))
    assert np.array_equal(C.sum(0), k * np.bincount(nxt.ravel(), minlength=E))
    assert C.sum() == 400 * k * k


def test_cooccurrence_golden():
    for case in GOLD["cooccurrence"]:
        E = case["E"]
        C = oracle.cooccurrence(np.array(case["prev"]), np.array(case["next"]), E)
        assert C.tolist() == case["C"], case["cite"]
        P = oracle.conditional(C.astype(np.int64))
        assert np.array_equal(P, np.array(case["P"], np.float32))
        ph = oracle.predict_next(np.array(case["p_seq_prev"], np.float32), P)
        assert np.array_equal(ph, np.array(case["p_hat"], np.float32))


def test_popularity_window_identities():
    """p_seq = Nw/sum(Nw): sums to one; with constant T it equals the mean of the
    per-iteration fractions exactly (both readings of the window average agree)."""
    rng = np.random.default_rng(21)
    E, T, k, s = 8, 64, 2, 10
    per_iter = []
    for it in range(s):
        idx, _ = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
        per_iter.append(oracle.histogram(idx, E))
    Nw = np.sum(per_iter, axis=0).astype(np.int64)
    p = oracle.popularity(Nw)
    assert abs(float(p.astype(np.float64).sum()) - 1.0) <= 1e-6
    for e in range(E):
        mean_frac = sum(Fraction(int(n[e]), T * k) for n in per_iter) / s
        assert p[e] == np.float32(float(mean_frac))
    assert np.all(oracle.popularity(np.zeros(E, np.int64)) == 0)


def test_conditional_rows_normalised():
    rng = np.random.default_rng(4)
    Cw = rng.integers(0, 50, size=(12, 12)).astype(np.int64)
    Cw[3] = 0
    P = oracle.conditional(Cw)
    sums = P.astype(np.float64).sum(1)
    assert np.all(np.abs(np.delete(sums, 3) - 1.0) <= 1e-6)
    assert np.all(P[3] == 0)
    assert np.array_equal(P[5], (Cw[5].astype(np.float32) / np.float32(Cw[5].sum())).astype(np.float32))


def test_prediction_end_of_window_identity():
    """Once layer l+1 has recorded the same iterations as layer l, propagating
    p_seq^l through P_l gives p_seq^{l+1} (the row normaliser k*Nw_l[a] cancels
    against p_seq^l[a] = Nw_l[a]/(k T_w) and the column sums are k*Nw_{l+1})."""
    cfg = synth.CONFIGS["tiny"]
    st = oracle.WindowStats(cfg.L, cfg.E, cfg.window)
    for it in range(13):
        prev = None
        for layer in range(cfg.L):
            lg = synth.logits(cfg, layer, it, None if prev is None else prev[:, 0])
            idx, _ = oracle.route(lg, cfg.k)
            st.record(layer, it, idx, prev)
            prev = idx
        p0, P0, _ = st.outputs(0)
        p1, _, _ = st.outputs(1)
        ph = oracle.predict_next(p0, P0)
        assert np.max(np.abs(ph.astype(np.float64) - p1)) <= 1e-6


def test_prediction_uses_causal_window():
    """Right after layer 0 records iteration it, pair (0,1) still holds it-window .. it-1."""
    E, k, window = 6, 2, 3
    st = oracle.WindowStats(2, E, window)
    rng = np.random.default_rng(8)
    hist = []
    for it in range(7):
        i0, _ = oracle.route(rng.standard_normal((50, E)).astype(np.float32), k)
        i1, _ = oracle.route(rng.standard_normal((50, E)).astype(np.float32), k)
        st.record(0, it, i0)
        _, P, _ = st.outputs(0)
        expect = sum((oracle.cooccurrence(a, b, E).astype(np.int64) for a, b in hist[-window:]),
                     np.zeros((E, E), np.int64))
        assert np.array_equal(P, oracle.conditional(expect))
        st.record(1, it, i1, i0)
        hist.append((i0, i1))


# --------------------------------------------------------------- replicas
def test_replicas_golden():
    for case in GOLD["replicas"]:
        r = oracle.replicas(np.array(case["counts"]), case["T"], case["k"], case["R"])
        assert r.tolist() == case["r"], case["cite"]


def test_replicas_closed_form_when_budget_does_not_bind():
    """MoE-GPS duplicate_experts with target T*k/E and threshold 1.0:
    copies = ceil(load/target) - 1 for load > target."""
    rng = np.random.default_rng(9)
    for trial in range(300):
        E = int(rng.integers(2, 12))
        T, k = int(rng.integers(4, 60)), int(rng.integers(1, min(E, 4) + 1))
        idx, _ = oracle.route(rng.standard_normal((T, E)).astype(np.float32) +
                              np.linspace(2, -2, E).astype(np.float32), k)
        n = oracle.histogram(idx, E)
        r = oracle.replicas(n, T, k, 10 ** 6)
        ref = [max(0, math.ceil(Fraction(int(ne) * E, T * k)) - 1) for ne in n]
        assert r.tolist() == ref


def test_replicas_bruteforce_minmax_when_budget_binds():
    rng = np.random.default_rng(10)
    for trial in range(150):
        E = int(rng.integers(2, 6))
        T, k = int(rng.integers(6, 30)), 1
        n = rng.multinomial(T * k, rng.dirichlet(np.ones(E) * 0.5)).astype(np.int32)
        R = int(rng.integers(1, 5))
        r = oracle.replicas(n, T, k, R)
        assert r.sum() <= R and np.all(r >= 0)
        unbound = [max(0, math.ceil(Fraction(int(ne) * E, T * k)) - 1) for ne in n]
        if sum(unbound) <= R:
            assert r.tolist() == unbound
            continue
        assert r.sum() == R
        got = max(Fraction(int(n[e]), int(r[e]) + 1) for e in range(E))
        best = min(max(Fraction(int(n[e]), a[e] + 1) for e in range(E))
                   for a in itertools.product(range(R + 1), repeat=E) if sum(a) <= R)
        assert got == best


# --------------------------------------------------------------- dispatch
def test_dispatch_golden():
    for case in GOLD["dispatch"]:
        d = oracle.dispatch(np.array(case["idx"]), case["E"], np.array(case["replicas"]))
        for key in ("expert_off", "perm_src", "inv_pos", "slot_off", "slot_expert"):
            assert np.asarray(d[key]).tolist() == case[key], (key, case["cite"])


@pytest.mark.parametrize("E,k,T", [(8, 2, 256), (160, 6, 300), (16, 4, 97)])
def test_dispatch_textbook_and_bijection(E, k, T):
    rng = np.random.default_rng(E * T)
    idx, _ = oracle.route(rng.standard_normal((T, E)).astype(np.float32) - np.log1p(np.arange(E)).astype(np.float32), k)
    n = oracle.histogram(idx, E)
    reps = oracle.replicas(n, T, k, 7)
    d = oracle.dispatch(idx, E, reps)
    assert np.array_equal(d["perm_src"], np.argsort(idx.ravel(), kind="stable") // k)
    assert np.array_equal(d["expert_off"], np.concatenate([[0], np.cumsum(n)]))
    flat = d["inv_pos"].ravel()
    assert np.array_equal(np.sort(flat), np.arange(T * k))                  # bijection
    assert np.array_equal(d["perm_src"][flat], np.repeat(np.arange(T), k))  # inv_pos o perm = id
    assert np.all(np.repeat(np.arange(E), n)[flat] == idx.ravel())          # row lies in its expert
    # replica chunks: contiguous, sizes differ by at most one, sum to n_e
    so, se = d["slot_off"], d["slot_expert"]
    assert d["n_slots"] == E + reps.sum() and so[-1] == T * k
    for e in range(E):
        sizes = np.diff(so)[se == e]
        assert len(sizes) == reps[e] + 1 and sizes.sum() == n[e] and sizes.max() - sizes.min() <= 1


def test_dispatch_duplicate_indices_follow_the_pair_order():
    """A token naming one expert twice (not a routing the top-k gate makes, but
    a valid permutation input): rows follow the stable order of the flattened
    (token, slot) pairs, so the token gets two rows of that expert in slot
    order -- the textbook stable argsort, checked against a brute-force walk."""
    rng = np.random.default_rng(11)
    T, k, E = 40, 3, 5
    idx = rng.integers(0, E, size=(T, k)).astype(np.int32)
    idx[0] = [2, 2, 2]
    idx[7] = [4, 1, 4]
    d = oracle.dispatch(idx, E)
    assert np.array_equal(d["perm_src"], np.argsort(idx.ravel(), kind="stable") // k)
    rows = [(e, t, i) for e in range(E) for t in range(T) for i in range(k) if idx[t, i] == e]
    brute = np.empty(T * k, np.int32)
    for r, (_, t, i) in enumerate(rows):
        brute[t * k + i] = r
    assert np.array_equal(d["inv_pos"].ravel(), brute)


def test_dispatch_empty_experts_and_no_replicas():
    idx = np.array([[3, 1]] * 5, np.int32)
    d = oracle.dispatch(idx, 6)
    assert d["expert_off"].tolist() == [0, 0, 5, 5, 10, 10, 10]
    assert d["slot_off"].tolist() == [0, 0, 5, 5, 10, 10, 10] and d["n_slots"] == 6


def test_permute_rows_bit_identical():
    x = synth.f32_to_bf16_bits(np.random.default_rng(1).standard_normal((33, 40)).astype(np.float32))
    perm = np.random.default_rng(2).integers(0, 33, size=70).astype(np.int32)
    assert np.array_equal(oracle.permute(x, perm), x[perm])


# ------------------------------------------------------------- expert FFN
def _np_ffn(x64, wg, wu, wd, act, rnd):
    z = x64 @ wg.T
    if act == "swiglu":
        a = z / (1.0 + np.exp(-z)) * (x64 @ wu.T)
    else:
        a = 0.5 * z * (1.0 + torch.erf(torch.from_numpy(z) / math.sqrt(2.0)).numpy())
    return rnd(rnd(a) @ wd.T)


def test_ffn_fp32_matches_numpy_fp64():
    rng = np.random.default_rng(5)
    E, H, I, n = 3, 48, 80, 20
    x = rng.standard_normal((n, H)).astype(np.float32)
    wg, wu, wd = (rng.standard_normal(s).astype(np.float32) / 7 for s in [(E, I, H), (E, I, H), (E, H, I)])
    ex = rng.integers(0, E, size=n).astype(np.int32)
    for act in ("swiglu", "gelu"):
        y = oracle.ffn_rows(x, ex, wg, wu if act == "swiglu" else None, wd, act)
        rnd = lambda v: v.astype(np.float32).astype(np.float64)
        for j in range(n):
            e = ex[j]
            ref = _np_ffn(x[j:j + 1].astype(np.float64), wg[e].astype(np.float64), wu[e].astype(np.float64),
                          wd[e].astype(np.float64), act, rnd)
            assert np.max(np.abs(y[j] - ref[0])) <= 1e-6 * max(1.0, np.max(np.abs(ref)))


def test_ffn_bf16_matches_numpy_fp64():
    rng = np.random.default_rng(6)
    E, H, I, n = 2, 32, 64, 12
    b = lambda a: synth.f32_to_bf16_bits(a.astype(np.float32))
    f = synth.bf16_bits_to_f32
    x = b(rng.standard_normal((n, H)))
    wg, wu, wd = (b(rng.standard_normal(s) / 5) for s in [(E, I, H), (E, I, H), (E, H, I)])
    ex = rng.integers(0, E, size=n).astype(np.int32)
    y = oracle.ffn_rows(x, ex, wg, wu, wd, "swiglu")
    rnd = lambda v: torch.from_numpy(np.asarray(v, np.float64)).to(torch.bfloat16).double().numpy()
    for j in range(n):
        e = ex[j]
        ref = _np_ffn(f(x[j:j + 1]).astype(np.float64), f(wg[e]).astype(np.float64), f(wu[e]).astype(np.float64),
                      f(wd[e]).astype(np.float64), "swiglu", rnd)
        got = f(y[j]).astype(np.float64)
        # one bf16 ulp of slack per element for a double-vs-single rounding of h
        assert np.all(np.abs(got - ref[0]) <= 2.0 ** -7 * np.abs(ref[0]) + 1e-30)


def test_bf16_rounding_matches_torch_on_fp32_values():
    rng = np.random.default_rng(7)
    v = rng.standard_normal(20000).astype(np.float32)
    v[:4] = np.array([1.00390625, 1.01171875, -1.00390625, 3.0e-39], np.float32)  # ties + subnormal
    ours = oracle.bf16_round_bits(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_single_expert_top1_is_dense_ffn():
    """E = 1, k = 1: the layer reduces to one dense FFN applied to every token."""
    rng = np.random.default_rng(13)
    T, H, I = 40, 32, 48
    x = rng.standard_normal((T, H)).astype(np.float32)
    wg, wu, wd = (rng.standard_normal(s).astype(np.float32) / 6 for s in [(1, I, H), (1, I, H), (1, H, I)])
    res = oracle.moe_layer(x, np.zeros((T, 1), np.float32), 1, (wg, wu, wd), "swiglu")
    assert np.all(res["w"] == 1.0)
    dense = oracle.ffn_rows(x, np.zeros(T, np.int32), wg, wu, wd, "swiglu")
    assert np.array_equal(res["out"], dense)


# ---------------------------------------------------------------- combine
def test_combine_golden():
    for case in GOLD["combine"]:
        out = oracle.combine(np.array(case["y_perm"], np.float32), np.array(case["inv_pos"]),
                             np.array(case["w"], np.float32))
        assert out.tolist() == case["out"], case["cite"]


def test_combine_k1_is_inverse_permutation():
    rng = np.random.default_rng(14)
    T, E, H = 64, 8, 16
    idx, w = oracle.route(rng.standard_normal((T, E)).astype(np.float32), 1)
    assert np.all(w == 1.0)
    d = oracle.dispatch(idx, E)
    y = rng.standard_normal((T, H)).astype(np.float32)
    out = oracle.combine(y, d["inv_pos"], w)
    assert np.array_equal(out, y[d["inv_pos"][:, 0]])


def test_combine_identity_experts_returns_input():
    rng = np.random.default_rng(15)
    T, E, k, H = 100, 8, 2, 24
    x = rng.standard_normal((T, H)).astype(np.float32)
    idx, w = oracle.route(rng.standard_normal((T, E)).astype(np.float32), k)
    d = oracle.dispatch(idx, E)
    out = oracle.combine(oracle.permute(x, d["perm_src"]), d["inv_pos"], w)
    assert np.max(np.abs(out - x)) <= 4 * 2.0 ** -24 * np.max(np.abs(x))


def test_replication_does_not_change_layer_output():
    cfg = synth.CONFIGS["tiny"]
    x = synth.hidden0(cfg, 0)
    lg = synth.logits(cfg, 0, 0)
    wts = synth.expert_weights(cfg)
    a = oracle.moe_layer(x, lg, cfg.k, wts, cfg.act)
    b = oracle.moe_layer(x, lg, cfg.k, wts, cfg.act, reps_budget=cfg.R)
    assert b["reps"].sum() == cfg.R
    assert np.array_equal(a["out"], b["out"])


def test_token_forward_matches_full_layer():
    cfg = synth.CONFIGS["tiny"]
    x = synth.hidden0(cfg, 1)
    lg = synth.logits(cfg, 0, 1)
    wts = synth.expert_weights(cfg)
    full = oracle.moe_layer(x, lg, cfg.k, wts, cfg.act)
    sample = np.array([0, 7, 100, 255])
    _, out = oracle.token_forward(x[sample], full["idx"][sample], full["w"][sample], wts, cfg.act)
    assert np.array_equal(out, full["out"][sample])


# ------------------------------------------------ replicas planned from a prediction
def _round_half_even(fr: Fraction) -> int:
    fl = math.floor(fr)
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def test_predicted_counts_exact_rational_rounding():
    """c_hat = p*total rounded half-to-even, checked in exact rational arithmetic
    (totals below 2^29 keep the double product exact)."""
    rng = np.random.default_rng(11)
    for trial in range(50):
        E = int(rng.integers(1, 40))
        total = int(rng.integers(0, 1 << 28))
        p = rng.random(E).astype(np.float32)
        got = oracle.predicted_counts(p, total)
        ref = [_round_half_even(Fraction(float(v)) * total) for v in p]
        assert got.tolist() == ref
    halves = np.array([0.5, 0.5, 0.25, 0.75], np.float32)
    assert oracle.predicted_counts(halves, 3).tolist() == [2, 2, 1, 2]   # 1.5->2, 0.75->1, 2.25->2
    assert oracle.predicted_counts(halves, 5).tolist() == [2, 2, 1, 4]   # 2.5->2, 1.25->1, 3.75->4
    odd = np.array([np.nan, -1.0, 0.0, np.inf, 3.0e9], np.float32)
    assert oracle.predicted_counts(odd, 1).tolist() == [0, 0, 0, 2147483647, 2147483647]


def test_plan_from_exact_shares_equals_plan_from_counts():
    """When the prediction is the exact share vector of some counts (a power-of-two
    total keeps n/total exact in fp32), the predicted plan is the counts plan."""
    rng = np.random.default_rng(12)
    for trial in range(40):
        E = int(rng.integers(2, 33))
        total = 1 << int(rng.integers(6, 16))
        cuts = np.sort(rng.integers(0, total + 1, size=E - 1))
        counts = np.diff(np.concatenate([[0], cuts, [total]])).astype(np.int32)
        p = (counts.astype(np.float64) / total).astype(np.float32)
        R = int(rng.integers(0, 2 * E))
        c_hat, r = oracle.plan_replicas(p, total, R)
        assert np.array_equal(c_hat, counts)
        assert np.array_equal(r, oracle.replicas(counts, total, 1, R))


def test_prediction_quality_hand_example():
    """counts 32/16/8/8 predicted exactly: tv 0, top-2 hit 1, loads (32,16,8,8) have
    std sqrt(96) and max/mean 2; one replica of expert 0 gives loads (16,16,16,8,8):
    mean 12.8, variance 15.36, max/mean 1.25."""
    p = np.array([0.5, 0.25, 0.125, 0.125], np.float32)
    n = np.array([32, 16, 8, 8], np.int32)
    q = oracle.prediction_quality(p, n, None, 2)
    assert q[0] == 0.0 and q[1] == 1.0
    assert q[2] == np.float32(math.sqrt(96.0)) and q[3] == 2.0
    q = oracle.prediction_quality(p, n, np.array([1, 0, 0, 0], np.int32), 2)
    assert q[2] == np.float32(math.sqrt(15.36)) and q[3] == np.float32(1.25)


def test_prediction_quality_against_independent_definitions():
    """tv in exact rationals, top-n by Python sorting, slot loads from the dispatch
    oracle's slot offsets with numpy's population std."""
    rng = np.random.default_rng(13)
    for trial in range(60):
        E = int(rng.integers(1, 24))
        k = int(rng.integers(1, min(E, 4) + 1))
        T = int(rng.integers(1, 300))
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        counts = oracle.histogram(idx, E)
        p = rng.random(E).astype(np.float32)
        if trial % 5 == 0:
            p[rng.integers(0, E)] = p.max()  # ties in the ranking
        reps = rng.integers(0, 3, size=E).astype(np.int32) if trial % 2 else None
        top_n = int(rng.integers(1, 7))
        q = oracle.prediction_quality(p, counts, reps, top_n)
        S = sum(Fraction(float(v)) for v in p)
        A = int(counts.sum())
        tv = sum(abs(Fraction(float(v)) / S - Fraction(int(c), A)) for v, c in zip(p, counts)) / 2
        assert abs(float(q[0]) - float(tv)) <= 2e-7 * max(1.0, float(tv))
        n = min(top_n, E)
        tp = set(sorted(range(E), key=lambda e: (-float(p[e]), e))[:n])
        tc = set(sorted(range(E), key=lambda e: (-int(counts[e]), e))[:n])
        assert q[1] == np.float32(len(tp & tc) / n)
        d = oracle.dispatch(idx, E, reps)
        loads = np.diff(d["slot_off"][: d["n_slots"] + 1]).astype(np.float64)
        assert len(loads) == E + (0 if reps is None else int(reps.sum()))
        assert abs(float(q[2]) - np.std(loads)) <= 1e-6 * max(1.0, np.std(loads))
        assert abs(float(q[3]) - loads.max() / loads.mean()) <= 1e-6 * loads.max() / loads.mean()


def test_prediction_quality_extremes():
    p = np.array([1.0, 0.0, 0.0], np.float32)
    n = np.array([0, 5, 7], np.int32)
    q = oracle.prediction_quality(p, n, None, 1)
    assert q[0] == 1.0 and q[1] == 0.0             # disjoint supports
    q = oracle.prediction_quality(np.zeros(3, np.float32), n, None, 3)
    assert q[0] == 1.0 and q[1] == 1.0             # no prediction mass; top-3 of 3 always hits
    q = oracle.prediction_quality(p, np.zeros(3, np.int32), None, 2)
    assert q[0] == 1.0 and q[2] == 0.0 and q[3] == 0.0


# ------------------------------------------------------------ window variants
def _rand_hist(rng, m, E, hi=5000):
    return rng.integers(0, hi, size=(m, E)).astype(np.int32)


def test_decayed_popularity_limits_are_plain_windows():
    """lambda = 1 is Eq.(1)'s plain window (bit-exact: the double quotient rounds to
    the same fp32 as the fp32 quotient of exact integers); lambda = 0 keeps only the
    current iteration."""
    rng = np.random.default_rng(21)
    for trial in range(40):
        m, E = int(rng.integers(1, 12)), int(rng.integers(1, 40))
        hist = _rand_hist(rng, m, E)
        assert np.array_equal(oracle.decayed_popularity(hist, 1.0), oracle.popularity(hist.sum(axis=0)))
        assert np.array_equal(oracle.decayed_popularity(hist, 0.0), oracle.popularity(hist[0].astype(np.int64)))


def test_decayed_popularity_exact_rationals():
    rng = np.random.default_rng(22)
    for trial in range(40):
        m, E = int(rng.integers(1, 12)), int(rng.integers(1, 20))
        lam = float(rng.choice([0.5, 0.75, 0.9, 0.99, 0.3]))
        hist = _rand_hist(rng, m, E)
        p = oracle.decayed_popularity(hist, lam)
        D = [sum(Fraction(lam) ** a * int(hist[a, e]) for a in range(m)) for e in range(E)]
        tot = sum(D)
        for e in range(E):
            ref = float(D[e] / tot) if tot else 0.0
            assert abs(float(p[e]) - ref) <= 6e-8 * max(ref, 1e-30) + 1e-45


def test_decayed_popularity_stationary_counts_ignore_lambda():
    """Identical counts in every iteration: every decay gives the same shares."""
    c = np.array([7, 0, 3, 90, 1], np.int32)
    hist = np.tile(c, (6, 1))
    ref = oracle.popularity(c.astype(np.int64))
    for lam in (0.0, 0.2, 0.9, 1.0):
        assert np.max(np.abs(oracle.decayed_popularity(hist, lam) - ref)) <= 1e-7


def test_load_anomalies_hand_cases():
    flags, summ = oracle.load_anomalies(np.array([[11, 10], [10, 10], [10, 10], [10, 10]], np.int32))
    assert flags.tolist() == [1, 0] and summ.tolist() == [1, 1]      # zero variance: any change flags
    flags, summ = oracle.load_anomalies(np.array([[5, 5, 5]], np.int32))
    assert flags.tolist() == [1, 1, 1] and summ.tolist() == [3, 1]   # no history yet
    flags, _ = oracle.load_anomalies(np.array([[4, 9], [4, 4], [4, 4]], np.int32))
    assert flags.tolist() == [0, 1]                                 # h = 2 is enough history
    # history 0, 10, 0, 10: mean 5, std 5; a load of 15 is at 2 std (not above), 16 is above
    h = np.array([[15, 16, 5], [0, 0, 0], [10, 10, 10], [0, 0, 0], [10, 10, 10]], np.int32)
    flags, summ = oracle.load_anomalies(h)
    assert flags.tolist() == [0, 1, 0] and summ.tolist() == [1, 1]
    E = 20
    h = np.tile(np.arange(E, dtype=np.int32), (5, 1))
    h[0, :4] += 1                                                    # 4 of 20 flagged: not transient
    assert oracle.load_anomalies(h)[1].tolist() == [4, 0]
    h[0, 4] += 1                                                     # 5 of 20: 5*5 > 20, transient
    assert oracle.load_anomalies(h)[1].tolist() == [5, 1]


def test_load_anomalies_exact_rationals():
    rng = np.random.default_rng(23)
    checked = 0
    for trial in range(60):
        m, E = int(rng.integers(3, 12)), int(rng.integers(1, 30))
        hist = _rand_hist(rng, m, E, hi=int(rng.choice([5, 100, 10000])))
        flags, summ = oracle.load_anomalies(hist)
        for e in range(E):
            hs = [Fraction(int(v)) for v in hist[1:, e]]
            mu = sum(hs) / len(hs)
            var = sum((v - mu) ** 2 for v in hs) / len(hs)
            lhs, rhs = (int(hist[0, e]) - mu) ** 2, 4 * var
            if lhs != rhs and abs(lhs - rhs) <= Fraction(1, 10 ** 9) * max(lhs, rhs):
                continue   # too close to call in double
            assert flags[e] == int(lhs > rhs)
            checked += 1
        assert summ[0] == flags.sum() and summ[1] == int(5 * flags.sum() > E)
    assert checked > 500


def test_window_history_matches_ring_order():
    ws = oracle.WindowStats(1, 3, 4)
    rng = np.random.default_rng(24)
    seen = []
    for it in range(7):
        idx = rng.integers(0, 3, size=(10, 1)).astype(np.int32)
        seen.append(oracle.histogram(idx, 3))
        ws.record(0, it, idx)
        hist = ws.history(0, it)
        assert hist.shape[0] == min(4, it + 1)
        for a in range(hist.shape[0]):
            assert np.array_equal(hist[a], seen[it - a])


# ------------------------------------------------------------------ backward
def _torch_layer_grads(x, logits, idx, weights, act, d_out):
    """Gradients by torch autograd in float64 of the forward written as plain tensor
    ops: kept-logit softmax, per-(token, slot) expert FFN, weighted sum."""
    f = lambda a: torch.tensor(synth.bf16_bits_to_f32(a) if a.dtype == np.uint16 else a, dtype=torch.float64,
                               requires_grad=True)
    X, Lg = f(x), torch.tensor(logits, dtype=torch.float64, requires_grad=True)
    Wg, Wd = f(weights[0]), f(weights[2])
    Wu = None if weights[1] is None else f(weights[1])
    it = torch.from_numpy(idx.astype(np.int64))
    w = torch.softmax(torch.gather(Lg, 1, it), dim=1)
    out = torch.zeros_like(X)
    for i in range(idx.shape[1]):
        e = it[:, i]
        if Wu is not None:
            h = torch.nn.functional.silu(torch.einsum("th,tih->ti", X, Wg[e])) * torch.einsum("th,tih->ti", X, Wu[e])
        else:
            z = torch.einsum("th,tih->ti", X, Wg[e])
            h = 0.5 * z * (1 + torch.erf(z / math.sqrt(2.0)))
        out = out + w[:, i:i + 1] * torch.einsum("ti,thi->th", h, Wd[e])
    dO = torch.tensor(synth.bf16_bits_to_f32(d_out) if d_out.dtype == np.uint16 else d_out, dtype=torch.float64)
    (out * dO).sum().backward()
    return dict(d_x=X.grad.numpy(), d_logits=Lg.grad.numpy(), d_w_gate=Wg.grad.numpy(),
                d_w_up=None if Wu is None else Wu.grad.numpy(), d_w_down=Wd.grad.numpy())


def _bw_case(name, T, seed):
    from oracle import backward as ob
    cfg = {"swiglu-f32": synth.CONFIGS["tiny"].scaled(T=T),
           "gelu-f32": synth.CONFIGS["popfetcher"].scaled(T=T, H=64, I=96, E=6, L=1),
           "swiglu-bf16": synth.CONFIGS["dbrx"].scaled(T=T, H=64, I=128, E=5)}[name]
    rng = np.random.default_rng(seed)
    x = synth.hidden0(cfg, seed)
    lg = synth.logits(cfg, 0, seed)
    idx, w = oracle.route(lg, cfg.k)
    wts = synth.expert_weights(cfg, 0)
    d_out = rng.standard_normal((cfg.T, cfg.H)).astype(np.float32)
    if cfg.dtype == "bf16":
        d_out = synth.f32_to_bf16_bits(d_out)
    return cfg, x, lg, idx, w, wts, d_out, ob.layer_backward(x, idx, w, wts, cfg.act, d_out)


@pytest.mark.parametrize("name", ["swiglu-f32", "gelu-f32", "swiglu-bf16"])
def test_backward_matches_torch_autograd_fp64(name):
    """An independent implementation of the gradients (torch autograd in float64 on
    plain tensor ops) agrees with the oracle's written-out chain rule to the
    dtype's rounding of the intermediates."""
    cfg, x, lg, idx, w, wts, d_out, got = _bw_case(name, 40, 5)
    ref = _torch_layer_grads(x, lg, idx, wts, cfg.act, d_out)
    tol = 1e-5 if cfg.dtype == "f32" else 2e-2
    for key in ("d_x", "d_w_gate", "d_w_up", "d_w_down", "d_logits"):
        if ref[key] is None:
            assert got[key] is None
            continue
        g = got[key]
        g = synth.bf16_bits_to_f32(g).astype(np.float64) if g.dtype == np.uint16 else g.astype(np.float64)
        rel = np.linalg.norm(g - ref[key]) / np.linalg.norm(ref[key])
        assert rel <= tol, (key, rel)


def test_backward_gate_invariants():
    """Softmax-Jacobian rows sum to zero; only kept experts get a logit gradient;
    a single expert (k = E = 1) has none at all."""
    cfg, x, lg, idx, w, wts, d_out, got = _bw_case("swiglu-f32", 64, 6)
    dl = got["d_logits"].astype(np.float64)
    assert np.all(np.abs(dl.sum(axis=1)) <= 1e-6 * (1 + np.abs(dl).sum(axis=1)))
    kept = np.zeros_like(dl, dtype=bool)
    np.put_along_axis(kept, idx.astype(np.int64), True, axis=1)
    assert np.all(dl[~kept] == 0)
    from oracle import backward as ob
    one = synth.CONFIGS["tiny"].scaled(T=16, E=1, k=1)
    x1, w1 = synth.hidden0(one, 0), synth.expert_weights(one, 0)
    i1, g1 = oracle.route(synth.logits(one, 0, 0), 1)
    r = ob.layer_backward(x1, i1, g1, w1, "swiglu", np.ones((16, one.H), np.float32))
    assert np.all(r["d_logits"] == 0)


def test_backward_is_linear_in_d_out():
    from oracle import backward as ob
    cfg, x, lg, idx, w, wts, d_out, got = _bw_case("gelu-f32", 24, 7)
    twice = ob.layer_backward(x, idx, w, wts, cfg.act, (2 * d_out).astype(np.float32))
    for key in ("d_x", "d_w_gate", "d_w_down"):
        assert np.array_equal(twice[key], 2 * got[key])   # power-of-two scaling is exact


@pytest.mark.parametrize("name", ["swiglu-f32", "gelu-f32", "swiglu-bf16"])
def test_sampled_backward_equals_full_backward(name):
    """The sampled form (for full-size checks) reproduces the whole-layer oracle."""
    from oracle import backward as ob
    cfg, x, lg, idx, w, wts, d_out, full = _bw_case(name, 48, 8)
    rng = np.random.default_rng(9)
    toks = rng.choice(cfg.T, size=7, replace=False)
    E, I, H = wts[0].shape
    entries = [("d_w_down", int(rng.integers(E)), int(rng.integers(H)), int(rng.integers(I))) for _ in range(6)]
    entries += [("d_w_gate", int(rng.integers(E)), int(rng.integers(I)), int(rng.integers(H))) for _ in range(6)]
    if wts[1] is not None:
        entries += [("d_w_up", int(rng.integers(E)), int(rng.integers(I)), int(rng.integers(H))) for _ in range(6)]
    dX, dL, vals = ob.sampled_backward(x, idx, w, wts, cfg.act, d_out, toks, entries)
    f64 = lambda a: synth.bf16_bits_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)
    tol = 1e-12 if cfg.dtype == "f32" else 0.0
    assert np.max(np.abs(dX - f64(full["d_x"])[toks])) <= tol + 1e-6 * np.max(np.abs(dX))
    assert np.max(np.abs(dL - full["d_logits"][toks])) <= 1e-6 * (1 + np.max(np.abs(dL)))
    for (nm, e, a, b), v in vals.items():
        ref = f64(full[nm])[e, a, b]
        assert abs(v - ref) <= 1e-6 * max(1.0, abs(ref)) + (4e-3 * abs(ref) if cfg.dtype == "bf16" else 0), (nm, e, a, b, v, ref)
