"""The seeded generator: deterministic bytes, workload shapes, skew and correlation recipe."""
import hashlib

import numpy as np
import torch

import synth


def _h(a):
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def test_same_seed_same_bytes():
    cfg = synth.CONFIGS["tiny"]
    assert _h(synth.logits(cfg, 0, 3)) == _h(synth.logits(cfg, 0, 3))
    assert _h(synth.hidden0(cfg, 2)) == _h(synth.hidden0(cfg, 2))
    a = synth.expert_weights(cfg)
    b = synth.expert_weights(cfg, threads=1)
    assert all(_h(x) == _h(y) for x, y in zip(a, b))
    assert _h(synth.logits(cfg, 0, 3)) != _h(synth.logits(cfg, 0, 4))


def test_weights_independent_of_T_and_subset():
    cfg = synth.CONFIGS["dsv2"].scaled(H=64, I=32)
    full = synth.expert_weights(cfg)
    part = synth.expert_weights(cfg.with_T(1024), experts=[3, 150])
    for f, p in zip(full, part):
        assert np.array_equal(f[[3, 150]], p[[3, 150]])


def test_bf16_bits_match_torch_rounding():
    v = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(v), ref)


def test_workload_shapes():
    c = synth.CONFIGS
    assert (c["mixtral"].T, c["mixtral"].H, c["mixtral"].I, c["mixtral"].E, c["mixtral"].k) == (8192, 4096, 14336, 8, 2)
    assert (c["dsv2"].E, c["dsv2"].k, c["dsv2"].H, c["dsv2"].I) == (160, 6, 5120, 1536)
    assert (c["dbrx"].E, c["dbrx"].k, c["dbrx"].H, c["dbrx"].I, c["dbrx"].R) == (16, 4, 6144, 10752, 16)
    p = c["popfetcher"]
    assert (p.L, p.H, p.I, p.E, p.k, p.T, p.window, p.act) == (12, 1024, 4096, 32, 2, 16384, 10, "gelu")


def test_bias_and_gamma_recipe():
    cfg = synth.CONFIGS["tiny"]
    rank = synth.expert_rank(cfg)
    assert np.allclose(synth.logit_bias(cfg), -1.0 * np.log(rank + 1.0), atol=1e-7)
    top1 = np.zeros(cfg.T, np.int64) + 3
    base = synth.logits(cfg.scaled(gamma=0.0), 1, 0)
    with_g = synth.logits(cfg, 1, 0, top1)
    diff = with_g - base
    col = synth.layer_pi(cfg, 0)[3]
    assert np.all(diff[:, col] == np.float32(2.0) + base[:, col] - base[:, col]) or np.allclose(diff[:, col], 2.0)
    assert np.all(np.delete(diff, col, axis=1) == 0)
