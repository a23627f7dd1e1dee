"""Seeded synthetic inputs for the MoE layer, shared by the oracle side and the HIP side.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no softmax, no selection, no counting, no GEMM).  Both the
oracle tests and the GPU path read the exact bytes produced here.

The workloads stand in for the real models and routing traces the pages measure
on (Mixtral 8x7B, DeepSeek-V2, DBRX and the MoE-GPT of PopFetcher; EPS-MoE
review, section 5 "experiments"; PopFetcher wiki, "experiments"), which are not
available.  Router logits follow a skewed-popularity recipe: N(0,1) noise plus a
per-expert bias -c*ln(rank_e+1) with a seeded rank permutation, so a few experts
are hot (PopFetcher wiki, observation 1: skewed, stable expert popularity).
Chained layers add gamma at a seeded permutation pi_l of the token's top-1
expert of the previous layer, which plants the layer-to-layer correlation that
PopFetcher's conditional probability (observation 2) measures.

Random streams: numpy PCG64 seeded by a SeedSequence of
[BASE, cfg, ..., tag, ...]; tags: rank=1, pi=2, noise=3, x0=4, w_gate/w1=5,
w_up=6, w_down/w2=7.  Weights do not depend on T, so a T sweep shares weights.
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

BASE_SEED = 20261203
TAG_RANK, TAG_PI, TAG_NOISE, TAG_X0, TAG_WG, TAG_WU, TAG_WD = 1, 2, 3, 4, 5, 6, 7


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    cfg: int            # config id, part of every seed
    T: int              # tokens per iteration
    H: int              # hidden size
    I: int              # expert FFN width
    E: int              # experts
    k: int              # top-k
    act: str            # "swiglu" | "gelu"
    dtype: str          # activation/weight dtype: "f32" | "bf16"
    L: int = 1          # chained MoE layers
    window: int = 10    # sliding-window length in iterations
    iters: int = 1      # iterations with fresh inputs
    R: int = 0          # replica budget (extra expert slots)
    c: float = 1.0      # popularity skew: bias_e = -c*ln(rank_e+1)
    gamma: float = 0.0  # layer-to-layer correlation strength

    def with_T(self, T: int) -> "Config":
        return dataclasses.replace(self, T=T)

    def scaled(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)

    @property
    def n_mat(self) -> int:
        return 3 if self.act == "swiglu" else 2

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4


# The five workloads.  Shapes of the real models are the ones the EPS-MoE
# review lists in its experiment setup (DeepSeekV2 160 experts top-6, Mixtral 8
# top-2, DBRX 16 top-4); PopFetcher's MoE-GPT uses H=1024.
CONFIGS = {
    "tiny": Config("tiny", 0, T=256, H=64, I=128, E=8, k=2, act="swiglu", dtype="f32",
                   L=2, window=10, iters=10, R=4, c=1.0, gamma=2.0),
    "mixtral": Config("mixtral", 1, T=8192, H=4096, I=14336, E=8, k=2, act="swiglu",
                      dtype="bf16", L=1, R=8, c=1.2),
    "dsv2": Config("dsv2", 2, T=4096, H=5120, I=1536, E=160, k=6, act="swiglu", dtype="bf16",
                   L=1, R=0, c=0.8),
    "dbrx": Config("dbrx", 3, T=4096, H=6144, I=10752, E=16, k=4, act="swiglu", dtype="bf16",
                   L=1, R=16, c=1.5),
    "popfetcher": Config("popfetcher", 4, T=16384, H=1024, I=4096, E=32, k=2, act="gelu",
                         dtype="f32", L=12, window=10, iters=10, R=0, c=1.0, gamma=1.5),
}
DSV2_T_SWEEP = (1024, 4096, 16384)


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([BASE_SEED, *key]))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (round-to-nearest-even) and return the uint16 bit patterns.
    Inputs are finite (synthetic normals), so no NaN handling is needed."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def expert_rank(cfg: Config) -> np.ndarray:
    """Seeded popularity rank of each expert (0 = most popular); shared by all layers."""
    return _rng(cfg.cfg, TAG_RANK).permutation(cfg.E)


def layer_pi(cfg: Config, layer: int) -> np.ndarray:
    """Seeded permutation pi_layer: a token whose top-1 at `layer` is x gets +gamma on
    expert pi_layer[x] at layer+1."""
    return _rng(cfg.cfg, TAG_PI, layer).permutation(cfg.E)


def logit_bias(cfg: Config) -> np.ndarray:
    rank = expert_rank(cfg).astype(np.float64)
    return (-cfg.c * np.log(rank + 1.0)).astype(np.float32)


def logits(cfg: Config, layer: int, it: int, prev_top1: np.ndarray | None = None) -> np.ndarray:
    """fp32 router logits [T, E] for `layer` at iteration `it`.

    Layer 0 (or gamma == 0): noise + bias.  Layer l > 0: also + gamma at column
    pi_{l-1}[prev_top1[t]], where prev_top1 is the caller's own top-1 of layer l-1."""
    noise = _rng(cfg.cfg, cfg.T, TAG_NOISE, layer, it).standard_normal((cfg.T, cfg.E), dtype=np.float32)
    out = noise + logit_bias(cfg)[None, :]
    if layer > 0 and cfg.gamma != 0.0:
        if prev_top1 is None:
            raise ValueError("layer > 0 needs the previous layer's top-1 expert per token")
        cols = layer_pi(cfg, layer - 1)[np.asarray(prev_top1, dtype=np.int64)]
        out[np.arange(cfg.T), cols] += np.float32(cfg.gamma)
    return np.ascontiguousarray(out, dtype=np.float32)


def hidden0(cfg: Config, it: int) -> np.ndarray:
    """Layer-0 hidden states [T, H], N(0,1).  fp32 array, or uint16 bf16 bits for bf16 configs."""
    x = _rng(cfg.cfg, cfg.T, TAG_X0, 0, it).standard_normal((cfg.T, cfg.H), dtype=np.float32)
    return f32_to_bf16_bits(x) if cfg.dtype == "bf16" else x


def _one_weight(cfg: Config, tag: int, layer: int, e: int, out_dim: int, in_dim: int) -> np.ndarray:
    w = _rng(cfg.cfg, tag, layer, e).standard_normal((out_dim, in_dim), dtype=np.float32)
    w *= np.float32(1.0 / math.sqrt(in_dim))
    return f32_to_bf16_bits(w) if cfg.dtype == "bf16" else w


def expert_weights(cfg: Config, layer: int = 0, experts=None, threads: int = 8):
    """Expert weights in nn.Linear [out, in] layout, stacked over experts.

    SwiGLU: (w_gate [E,I,H], w_up [E,I,H], w_down [E,H,I]).
    GELU:   (w1 [E,I,H], None, w2 [E,H,I]).
    std = 1/sqrt(fan_in): fan_in = H for gate/up/w1, I for down/w2.
    `experts` restricts generation to a subset (rows of the other experts are zero)."""
    E, H, I = cfg.E, cfg.H, cfg.I
    dt = np.uint16 if cfg.dtype == "bf16" else np.float32
    sel = range(E) if experts is None else sorted(set(int(e) for e in experts))
    mats = [("g", TAG_WG, I, H)]
    if cfg.act == "swiglu":
        mats.append(("u", TAG_WU, I, H))
    mats.append(("d", TAG_WD, H, I))
    out = {name: np.zeros((E, o, i), dtype=dt) for name, _, o, i in mats}
    jobs = [(name, tag, o, i, e) for name, tag, o, i in mats for e in sel]

    def run(job):
        name, tag, o, i, e = job
        out[name][e] = _one_weight(cfg, tag, layer, e, o, i)

    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(run, jobs))
    return out["g"], out.get("u"), out["d"]


def tie_logits(T: int, E: int, seed: int = 7) -> np.ndarray:
    """Logits drawn from the 9 values {-2,-1.5,...,2}: ties between experts are frequent,
    which exercises the lowest-index tie rule (N(0,1) floats almost never tie)."""
    r = _rng(99, seed, T, E).integers(-4, 5, size=(T, E))
    return np.ascontiguousarray(r.astype(np.float32) * np.float32(0.5))
