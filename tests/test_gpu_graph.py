"""The layer forward captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

A small batch is launch-bound: its kernels take a few microseconds each, about
what the host needs to issue them.  A graph replay issues a whole chain of
layers with one call.  The grouped path enqueues no host synchronisation and
no memset (the statistics and tile tables clear their counters with kernels),
so it can be captured.  Every replay must equal the eager chain bit for bit:
the replays are interleaved with unrelated eager work and synchronisations,
and the statistics of one iteration index are idempotent (a replay writes the
same ring slot with the same counts, so the window sums do not move)."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_top_amd as moe
import synth
from _util import to_dev

pytestmark = pytest.mark.gpu


def _chain(cfg):
    L, E, k, win = cfg.L, cfg.E, cfg.k, cfg.window
    weights = [tuple(None if w is None else to_dev(w) for w in synth.expert_weights(cfg, l)) for l in range(L)]
    state = torch.empty(moe.moe_stats_state_bytes(L, E, win), dtype=torch.uint8, device="cuda")
    moe.moe_stats_init(state, L, E, win)
    x0 = to_dev(synth.hidden0(cfg, 0))
    # chained logits from the GPU's own routing of the previous layer
    lgs, prev = [], None
    for l in range(L):
        lgs.append(to_dev(synth.logits(cfg, l, 0, prev)))
        prev = moe.moe_route(lgs[-1], k)[0][:, 0].cpu().numpy()
    bufs = [dict() for _ in range(L)]

    def run(it):
        xx, prev_idx, res = x0, None, []
        for l in range(L):
            r = moe.moe_layer_forward(xx, lgs[l], k, *weights[l], cfg.act, cfg.R, stats_state=state,
                                      stats_dims=(L, E, win), layer=l, it=it, prev_topk_idx=prev_idx, bufs=bufs[l])
            res.append(r)
            xx, prev_idx = r["out"], r["idx"]
        return res
    return run


def _snapshot(res):
    keys = ("out", "idx", "w", "counts", "p_seq", "replicas", "perm_src", "inv_pos", "slot_off", "cond", "pred_next")
    return [{kk: r[kk].clone() for kk in keys if kk in r and r[kk] is not None} for r in res]


@pytest.mark.parametrize("name", ["tiny", "chain-bf16"])
def test_layer_chain_graph_replay_matches_eager(name):
    cfg = synth.CONFIGS["tiny"] if name == "tiny" else \
        synth.CONFIGS["dbrx"].scaled(T=384, H=256, I=320, L=3, window=4, R=6, gamma=1.5)
    run = _chain(cfg)
    it = 5
    run(it)                       # allocates every buffer the chain reuses
    eager = _snapshot(run(it))    # the same iteration again: the reference
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(it)                   # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = run(it)
    for rep in range(3):
        for r in captured:        # scribble over the outputs the replay must rewrite
            r["out"].fill_(-7.0)
        assert float(torch.randn(4096, device="cuda").abs().sum()) > 0   # eager work, then a sync
        graph.replay()
        torch.cuda.synchronize()
        got = _snapshot(captured)
        for layer, (g, e) in enumerate(zip(got, eager)):
            for kk in e:
                assert torch.equal(g[kk], e[kk]), (name, rep, layer, kk)
