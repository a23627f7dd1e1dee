"""GPU parity of the planning calls: replicas planned from a predicted
distribution (moe_plan_replicas) and the prediction-quality measures
(moe_prediction_quality), against the CPU oracle on the same inputs, alone and
inside the statistics chain whose prediction feeds them."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_top_amd as moe
import oracle
import synth
from _util import from_dev, to_dev

pytestmark = pytest.mark.gpu


def _sync():
    torch.cuda.synchronize()


def _rand_pred(rng, E, kind):
    if kind == "dirichlet":
        return rng.dirichlet(np.full(E, 0.3)).astype(np.float32)
    if kind == "halves":  # p * total lands on .5 for many experts
        return (rng.integers(0, 8, size=E) / 16.0).astype(np.float32)
    p = rng.random(E).astype(np.float32)
    p[rng.integers(0, E, size=max(1, E // 8))] = np.float32(np.nan)
    p[rng.integers(0, E, size=max(1, E // 8))] = -0.25
    p[rng.integers(0, E)] = np.inf
    return p


@pytest.mark.parametrize("E", [1, 5, 8, 32, 160, 256])
@pytest.mark.parametrize("kind", ["dirichlet", "halves", "odd"])
def test_plan_replicas_matches_oracle(E, kind):
    rng = np.random.default_rng(E * 7 + len(kind))
    for total, R in [(0, 4), (8, 3), (16384 * 2, 8), (4096 * 6, 64), ((1 << 31) - 1, 4096), (1000, 0)]:
        p = _rand_pred(rng, E, kind)
        c_g, r_g = moe.moe_plan_replicas(to_dev(p), total, R)
        _sync()
        c_o, r_o = oracle.plan_replicas(p, total, R)
        assert np.array_equal(from_dev(c_g), c_o), (total, R)
        assert np.array_equal(from_dev(r_g), r_o), (total, R)


@pytest.mark.parametrize("E", [1, 3, 8, 32, 160, 256])
def test_prediction_quality_matches_oracle(E):
    rng = np.random.default_rng(100 + E)
    for trial in range(8):
        p = rng.random(E).astype(np.float32)
        if trial % 2:
            p[rng.integers(0, E, size=max(1, E // 3))] = p.max()   # ties in the ranking
        counts = rng.integers(0, 500, size=E).astype(np.int32)
        if trial == 3:
            counts[:] = 0
        if trial == 5:
            p[:] = 0
        reps = rng.integers(0, 4, size=E).astype(np.int32) if trial % 3 else None
        if trial == 7 and reps is not None:
            reps[0] = 1 << 20                                       # clamped to 4096
        top_n = int(rng.integers(1, 9))
        q_g = moe.moe_prediction_quality(to_dev(p), to_dev(counts), None if reps is None else to_dev(reps), top_n)
        _sync()
        q_o = oracle.prediction_quality(p, counts, reps, top_n)
        q_g = from_dev(q_g)
        assert q_g[1] == q_o[1], trial
        for j in (0, 2, 3):
            assert abs(float(q_g[j]) - float(q_o[j])) <= 1e-6 * max(1.0, abs(float(q_o[j]))), (trial, j, q_g, q_o)


@pytest.mark.parametrize("name,iters,R", [("tiny", 12, 4), ("popfetcher", 10, 8)])
def test_predictive_chain_matches_oracle(name, iters, R):
    """Each layer l >= 1 is planned from layer l-1's prediction before it routes;
    after it routes, the plan and the prediction are scored against its counts."""
    cfg = synth.CONFIGS[name]
    L, E, k, win, T = cfg.L, cfg.E, cfg.k, cfg.window, cfg.T
    state = torch.empty(moe.moe_stats_state_bytes(L, E, win), dtype=torch.uint8, device="cuda")
    moe.moe_stats_init(state, L, E, win)
    ost = oracle.WindowStats(L, E, win)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    pred = torch.empty(E, dtype=torch.float32, device="cuda")
    scored = 0
    for it in range(iters):
        prev_o, prev_g, plan_g, pred_o, plan_o, pred_g = None, None, None, None, None, None
        for layer in range(L):
            lg = synth.logits(cfg, layer, it, None if prev_o is None else prev_o[:, 0])
            idx_g, _ = moe.moe_route(to_dev(lg), k)
            last = layer + 1 >= L
            moe.moe_stats(state, L, E, win, layer, it, idx_g, prev_g, k, counts, None, None,
                          None if last else pred)
            idx_o, _ = oracle.route(lg, k)
            cnt = ost.record(layer, it, idx_o, prev_o)
            if plan_g is not None:
                q_g = from_dev(moe.moe_prediction_quality(pred_g, counts, plan_g, 5))
                q_o = oracle.prediction_quality(pred_o, cnt, plan_o, 5)
                assert q_g[1] == q_o[1]
                assert np.max(np.abs(q_g - q_o) / np.maximum(1.0, np.abs(q_o))) <= 1e-6, (it, layer, q_g, q_o)
                scored += 1
            if not last:
                pred_g = pred.clone()
                _, plan_g = moe.moe_plan_replicas(pred_g, T * k, R)
                _sync()
                pred_o = ost.outputs(layer)[2]
                assert np.array_equal(from_dev(pred_g), pred_o), (it, layer)   # same double sums
                _, plan_o = oracle.plan_replicas(pred_o, T * k, R)
                assert np.array_equal(from_dev(plan_g), plan_o), (it, layer)
            prev_o, prev_g = idx_o, idx_g
    assert scored == iters * (L - 1)


def test_layer_forward_with_planned_replicas_is_bit_identical():
    """A plan from the prediction only moves rows between slots: the layer output
    equals the unreplicated one bit for bit, and the slots follow the plan."""
    cfg = synth.CONFIGS["popfetcher"].scaled(T=500, H=128, I=256, L=1)
    E, k, R = cfg.E, cfg.k, 6
    x = synth.hidden0(cfg, 0)
    lg = synth.logits(cfg, 0, 0)
    wts = synth.expert_weights(cfg, 0)
    wg, wu, wd = (None if w is None else to_dev(w) for w in wts)
    skew = np.float32(1.0) / (1 + np.arange(E, dtype=np.float32))
    pred = (skew / skew.sum()).astype(np.float32)
    _, plan = moe.moe_plan_replicas(to_dev(pred), cfg.T * k, R)
    base = moe.moe_layer_forward(to_dev(x), to_dev(lg), k, wg, wu, wd, cfg.act, 0)
    out0 = from_dev(base["out"]).copy()
    res = moe.moe_layer_forward(to_dev(x), to_dev(lg), k, wg, wu, wd, cfg.act, R, planned_replicas=plan)
    _sync()
    plan_np = from_dev(plan)
    assert plan_np.sum() > 0
    assert int(from_dev(res["n_slots"])[0]) == E + int(plan_np.sum())
    ref = oracle.dispatch(oracle.route(lg, k)[0], E, plan_np)
    assert np.array_equal(from_dev(res["slot_off"])[: ref["n_slots"] + 1], ref["slot_off"])
    assert np.array_equal(from_dev(res["out"]), out0)
