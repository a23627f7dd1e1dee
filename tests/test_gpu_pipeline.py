"""The horizontally split layer (moe_layer_forward_pipelined): chunks of tokens
pipelined over a memory stream and a compute stream must give the unsplit
layer's output bit for bit, for any chunk count, with cached buffers reused."""
import numpy as np
import pytest
import torch

import mixture_experts_routing_top_amd as moe
import oracle
import synth
from _util import assert_close, from_dev, to_dev

pytestmark = pytest.mark.gpu

MINI = {
    "mixtral-mini": synth.CONFIGS["mixtral"].scaled(T=300, H=256, I=448),
    "dsv2-mini": synth.CONFIGS["dsv2"].scaled(T=200, H=320, I=192),
    "popf-mini": synth.CONFIGS["popfetcher"].scaled(T=500, H=128, I=256, L=1),
}


@pytest.mark.parametrize("name", list(MINI))
@pytest.mark.parametrize("two_streams", [False, True])
def test_pipelined_layer_is_bit_identical(name, two_streams):
    cfg = MINI[name]
    wts = synth.expert_weights(cfg, 0)
    wg, wu, wd = (None if w is None else to_dev(w) for w in wts)
    cs = torch.cuda.current_stream()
    ms = torch.cuda.Stream() if two_streams else cs
    bufs = {}
    for it in range(2):
        x = to_dev(synth.hidden0(cfg, it))
        lg = to_dev(synth.logits(cfg, 0, it))
        ref = from_dev(moe.moe_layer_forward(x, lg, cfg.k, wg, wu, wd, cfg.act, 0)["out"]).copy()
        for n in (1, 2, 3, 5):
            res = moe.moe_layer_forward_pipelined(x, lg, cfg.k, wg, wu, wd, cfg.act, n, cs, ms, bufs)
            torch.cuda.synchronize()
            assert np.array_equal(from_dev(res["out"]), ref), (it, n)
    # and against the oracle on sampled tokens of the last call
    xs = synth.hidden0(cfg, 1)
    ridx, rw = oracle.route(synth.logits(cfg, 0, 1), cfg.k)
    rows = np.arange(0, cfg.T, 37)
    got = from_dev(res["out"])[rows]
    _, ref_rows = oracle.token_forward(xs[rows], ridx[rows], rw[rows], wts, cfg.act)
    assert_close(got, ref_rows, "bf16" if cfg.dtype == "bf16" else "fp32_gemm", name)


def test_pipelined_more_chunks_than_tokens():
    cfg = MINI["popf-mini"].scaled(T=3)
    wts = synth.expert_weights(cfg, 0)
    wg, wu, wd = (None if w is None else to_dev(w) for w in wts)
    x, lg = to_dev(synth.hidden0(cfg, 0)), to_dev(synth.logits(cfg, 0, 0))
    ref = from_dev(moe.moe_layer_forward(x, lg, cfg.k, wg, wu, wd, cfg.act, 0)["out"]).copy()
    res = moe.moe_layer_forward_pipelined(x, lg, cfg.k, wg, wu, wd, cfg.act, 8, None, torch.cuda.Stream())
    torch.cuda.synchronize()
    assert np.array_equal(from_dev(res["out"]), ref)
