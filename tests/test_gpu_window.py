"""GPU parity of the window variants (moe_stats_load_state): decayed-window
popularity, per-expert anomaly flags and the transient/stable state, against
the CPU oracle on the count ring of the same routed chains."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_top_amd as moe
import oracle
import synth
from _util import from_dev, to_dev

pytestmark = pytest.mark.gpu

DECAYS = (0.0, 0.5, 0.9, 1.0)


def _chain(cfg, iters, logits_cfg=None):
    """Route and record a chain on both sides; after every layer compare the
    window variants for several decays.  logits_cfg(it) may swap the workload
    (a drift in expert popularity)."""
    L, E, k, win = cfg.L, cfg.E, cfg.k, cfg.window
    state = torch.empty(moe.moe_stats_state_bytes(L, E, win), dtype=torch.uint8, device="cuda")
    moe.moe_stats_init(state, L, E, win)
    ost = oracle.WindowStats(L, E, win)
    p_seq = torch.empty(E, dtype=torch.float32, device="cuda")
    states = []
    for it in range(iters):
        c = cfg if logits_cfg is None else logits_cfg(it)
        prev_o, prev_g = None, None
        for layer in range(L):
            lg = synth.logits(c, layer, it, None if prev_o is None else prev_o[:, 0])
            idx_g, _ = moe.moe_route(to_dev(lg), k)
            moe.moe_stats(state, L, E, win, layer, it, idx_g, prev_g, k, None, p_seq)
            idx_o, _ = oracle.route(lg, k)
            ost.record(layer, it, idx_o, prev_o)
            hist = ost.history(layer, it)
            for decay in DECAYS:
                r = moe.moe_stats_load_state(state, L, E, win, layer, it, decay)
                torch.cuda.synchronize()
                assert np.array_equal(from_dev(r["p_decay"]), oracle.decayed_popularity(hist, decay)), (it, layer, decay)
                flags, summ = oracle.load_anomalies(hist)
                assert np.array_equal(from_dev(r["anomalous"]), flags), (it, layer)
                assert np.array_equal(from_dev(r["summary"]), summ), (it, layer)
                if decay == 1.0:   # the plain window of moe_stats
                    assert np.array_equal(from_dev(r["p_decay"]), from_dev(p_seq))
            states.append((it, layer, int(summ[1]), int(summ[0])))
            prev_o, prev_g = idx_o, idx_g
    return states


def test_window_variants_tiny_chain_wraps_ring():
    _chain(synth.CONFIGS["tiny"], 13)


def test_window_variants_popfetcher_chain():
    cfg = synth.CONFIGS["popfetcher"].scaled(T=4096)
    _chain(cfg, 6)


def test_window_variants_large_E():
    _chain(synth.CONFIGS["dsv2"].scaled(T=1024, window=4), 6)


def test_popularity_drift_turns_layer_transient():
    """Stable skewed routing for 8 iterations, then the expert ranking changes:
    the iteration after the change is flagged transient by both sides."""
    base = synth.CONFIGS["popfetcher"].scaled(T=8192, L=1, c=1.5)
    drifted = base.scaled(cfg=40)    # another seed: another popularity ranking
    states = _chain(base, 11, lambda it: base if it < 8 else drifted)
    by_it = {it: (tr, n) for it, _, tr, n in states}
    assert by_it[8][0] == 1 and by_it[8][1] > base.E // 2
    assert all(by_it[it][0] == 0 for it in (5, 6, 7))
