"""CPU oracle for the MoE layer forward pass -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the CPU-baseline leg of the benchmark may
import this package.  The arithmetic lives in moe_oracle.c (plain C, single
thread, double accumulation); this module compiles it with gcc, marshals numpy
arrays through ctypes, and keeps the sliding-window ring for the statistics.
It shares no code with the HIP library and never imports it.

Every function here has a pin in tests/test_oracle_pins.py (textbook
routines, closed forms, invariants, brute force on tiny inputs).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

F32, BF16 = 0, 1
SWIGLU, GELU = 0, 1


def build(force: bool = True) -> str:
    """Compile moe_oracle.c into liboracle.so (gcc -O2, IEEE semantics, no fast-math)."""
    global _lib
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-fPIC", "-shared", "-fno-fast-math",
                               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
        _lib = None
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_LIB_PATH)
        for name in ("oracle_route", "oracle_histogram", "oracle_cooccurrence", "oracle_popularity",
                     "oracle_conditional", "oracle_predict_next", "oracle_replicas", "oracle_dispatch",
                     "oracle_predicted_counts", "oracle_plan_replicas", "oracle_prediction_quality",
                     "oracle_decayed_popularity", "oracle_load_anomalies",
                     "oracle_permute", "oracle_ffn_rows", "oracle_combine", "oracle_bf16_round_bits"):
            getattr(_lib, name).restype = ctypes.c_int
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _i64(v):
    return ctypes.c_int64(int(v))


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its input (rc={rc})")


def _dt_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    raise TypeError("activations must be float32 or uint16 bf16 bits")


# ------------------------------------------------------------------ routing
def route(logits: np.ndarray, k: int):
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    T, E = logits.shape
    idx = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _check(lib().oracle_route(_p(logits), _i64(T), E, k, _p(idx), _p(w)), "route")
    return idx, w


# --------------------------------------------------------------- statistics
def histogram(idx: np.ndarray, E: int) -> np.ndarray:
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    out = np.empty(E, np.int32)
    _check(lib().oracle_histogram(_p(idx), _i64(T), k, E, _p(out)), "histogram")
    return out


def cooccurrence(prev: np.ndarray, nxt: np.ndarray, E: int) -> np.ndarray:
    prev = np.ascontiguousarray(prev, dtype=np.int32)
    nxt = np.ascontiguousarray(nxt, dtype=np.int32)
    T, k = prev.shape
    C = np.empty((E, E), np.int32)
    _check(lib().oracle_cooccurrence(_p(prev), _p(nxt), _i64(T), k, E, _p(C)), "cooccurrence")
    return C


def popularity(Nw: np.ndarray) -> np.ndarray:
    Nw = np.ascontiguousarray(Nw, dtype=np.int64)
    p = np.empty(Nw.shape[0], np.float32)
    lib().oracle_popularity(_p(Nw), Nw.shape[0], _p(p))
    return p


def conditional(Cw: np.ndarray) -> np.ndarray:
    Cw = np.ascontiguousarray(Cw, dtype=np.int64)
    E = Cw.shape[0]
    P = np.empty((E, E), np.float32)
    lib().oracle_conditional(_p(Cw), E, _p(P))
    return P


def predict_next(p_seq: np.ndarray, P: np.ndarray) -> np.ndarray:
    p_seq = np.ascontiguousarray(p_seq, dtype=np.float32)
    P = np.ascontiguousarray(P, dtype=np.float32)
    out = np.empty(p_seq.shape[0], np.float32)
    lib().oracle_predict_next(_p(p_seq), _p(P), p_seq.shape[0], _p(out))
    return out


def replicas(counts: np.ndarray, T: int, k: int, R: int) -> np.ndarray:
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    r = np.empty(counts.shape[0], np.int32)
    lib().oracle_replicas(_p(counts), counts.shape[0], _i64(T), k, R, _p(r))
    return r


def predicted_counts(p_hat: np.ndarray, total: int) -> np.ndarray:
    p_hat = np.ascontiguousarray(p_hat, dtype=np.float32)
    out = np.empty(p_hat.shape[0], np.int32)
    lib().oracle_predicted_counts(_p(p_hat), p_hat.shape[0], _i64(total), _p(out))
    return out


def plan_replicas(p_hat: np.ndarray, total: int, R: int):
    """(predicted counts, replicas) planned from a predicted distribution."""
    p_hat = np.ascontiguousarray(p_hat, dtype=np.float32)
    E = p_hat.shape[0]
    c_hat = np.empty(E, np.int32)
    r = np.empty(E, np.int32)
    _check(lib().oracle_plan_replicas(_p(p_hat), E, _i64(total), R, _p(c_hat), _p(r)), "plan_replicas")
    return c_hat, r


def prediction_quality(p_hat: np.ndarray, counts: np.ndarray, reps: np.ndarray | None, top_n: int) -> np.ndarray:
    """[tv distance, top-n hit rate, slot-load std, max/mean slot load] as float32."""
    p_hat = np.ascontiguousarray(p_hat, dtype=np.float32)
    counts = np.ascontiguousarray(counts, dtype=np.int32)
    out = np.empty(4, np.float32)
    rp = None if reps is None else np.ascontiguousarray(reps, dtype=np.int32)
    _check(lib().oracle_prediction_quality(_p(p_hat), _p(counts), p_hat.shape[0],
                                           None if rp is None else _p(rp), top_n, _p(out)), "prediction_quality")
    return out


def decayed_popularity(hist: np.ndarray, lam: float) -> np.ndarray:
    """hist [m, E] youngest first (row 0 = the current iteration)."""
    hist = np.ascontiguousarray(hist, dtype=np.int32)
    m, E = hist.shape
    p = np.empty(E, np.float32)
    lib().oracle_decayed_popularity(_p(hist), m, E, ctypes.c_double(lam), _p(p))
    return p


def load_anomalies(hist: np.ndarray):
    """(flags int32 [E], [n_flagged, transient]) for hist [m, E] youngest first."""
    hist = np.ascontiguousarray(hist, dtype=np.int32)
    m, E = hist.shape
    flags = np.empty(E, np.int32)
    summary = np.empty(2, np.int32)
    lib().oracle_load_anomalies(_p(hist), m, E, _p(flags), _p(summary))
    return flags, summary


class WindowStats:
    """The sliding-window statistics state of a chain of L MoE layers.

    Recording layer l at iteration it replaces ring slot it % window of layer
    l's counts, and (l > 0) of pair (l-1, l)'s co-occurrence.  The window is the
    sum over the ring.  Right after layer l is recorded, its popularity covers
    the last `window` iterations up to `it`, while pair (l, l+1) still holds
    iterations it-window .. it-1 (layer l+1 has not run at `it`): the
    prediction for layer l+1 is causal (PopFetcher's prediction precedes the
    layer it prepares)."""

    def __init__(self, L: int, E: int, window: int):
        self.L, self.E, self.window = L, E, window
        self.cnt = np.zeros((window, L, E), np.int64)
        self.cooc = np.zeros((window, max(L - 1, 0), E, E), np.int64)

    def record(self, layer: int, it: int, idx: np.ndarray, prev_idx: np.ndarray | None = None):
        s = it % self.window
        self.cnt[s, layer] = histogram(idx, self.E)
        if layer > 0:
            if prev_idx is None:
                raise ValueError("layer > 0 needs the previous layer's routing")
            self.cooc[s, layer - 1] = cooccurrence(prev_idx, idx, self.E)
        return self.cnt[s, layer].astype(np.int32)

    def history(self, layer: int, it: int) -> np.ndarray:
        """The recorded counts of `layer` for iterations it, it-1, ... still in the
        window (youngest first): [min(window, it+1), E]."""
        m = min(self.window, it + 1)
        return np.stack([self.cnt[(it - a) % self.window, layer] for a in range(m)]).astype(np.int32)

    def window_counts(self, layer: int) -> np.ndarray:
        return self.cnt[:, layer].sum(axis=0)

    def window_cooc(self, pair: int) -> np.ndarray:
        return self.cooc[:, pair].sum(axis=0)

    def outputs(self, layer: int):
        """(p_seq of `layer`, P of pair (layer, layer+1) or None, p_hat for layer+1 or None)."""
        p = popularity(self.window_counts(layer))
        if layer + 1 >= self.L:
            return p, None, None
        P = conditional(self.window_cooc(layer))
        return p, P, predict_next(p, P)


# ----------------------------------------------------------------- dispatch
def dispatch(idx: np.ndarray, E: int, reps: np.ndarray | None = None):
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T, k = idx.shape
    M = T * k
    S = E + (int(np.sum(reps)) if reps is not None else 0)
    expert_off = np.empty(E + 1, np.int32)
    perm_src = np.empty(M, np.int32)
    inv_pos = np.empty(M, np.int32)
    slot_off = np.empty(S + 1, np.int32)
    slot_expert = np.empty(max(S, 1), np.int32)
    n_slots = np.zeros(1, np.int32)
    rp = None if reps is None else np.ascontiguousarray(reps, dtype=np.int32)
    _check(lib().oracle_dispatch(_p(idx), _i64(T), k, E, None if rp is None else _p(rp), _p(expert_off),
                                 _p(perm_src), _p(inv_pos), _p(slot_off), _p(slot_expert), _p(n_slots)),
           "dispatch")
    return dict(expert_off=expert_off, perm_src=perm_src, inv_pos=inv_pos.reshape(T, k),
                slot_off=slot_off, slot_expert=slot_expert[:S], n_slots=int(n_slots[0]))


def permute(x: np.ndarray, perm_src: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x)
    perm_src = np.ascontiguousarray(perm_src, dtype=np.int32)
    out = np.empty((perm_src.shape[0],) + x.shape[1:], x.dtype)
    row_bytes = x.strides[0]
    _check(lib().oracle_permute(_p(x), _i64(x.shape[0]), _i64(row_bytes), _p(perm_src),
                                _i64(perm_src.shape[0]), _p(out)), "permute")
    return out


# --------------------------------------------------------------- expert FFN
def ffn_rows(x: np.ndarray, experts: np.ndarray, w_gate, w_up, w_down, act: str) -> np.ndarray:
    """y[j] = FFN_{experts[j]}(x[j]) for independent rows (fp32 or bf16-bit arrays)."""
    x = np.ascontiguousarray(x)
    dt = _dt_code(x)
    n, H = x.shape
    E, I, _ = w_gate.shape
    experts = np.ascontiguousarray(experts, dtype=np.int32)
    y = np.empty((n, H), x.dtype)
    a = SWIGLU if act == "swiglu" else GELU
    wu = None if w_up is None else _p(np.ascontiguousarray(w_up))
    _check(lib().oracle_ffn_rows(_p(x), dt, _i64(n), H, I, _p(experts), E, _p(np.ascontiguousarray(w_gate)),
                                 wu, _p(np.ascontiguousarray(w_down)), a, _p(y)), "ffn_rows")
    return y


def combine(y_perm: np.ndarray, inv_pos: np.ndarray, w: np.ndarray) -> np.ndarray:
    y_perm = np.ascontiguousarray(y_perm)
    dt = _dt_code(y_perm)
    inv_pos = np.ascontiguousarray(inv_pos, dtype=np.int32)
    w = np.ascontiguousarray(w, dtype=np.float32)
    T, k = w.shape
    H = y_perm.shape[1]
    out = np.empty((T, H), y_perm.dtype)
    _check(lib().oracle_combine(_p(y_perm), dt, _i64(y_perm.shape[0]), _p(inv_pos), _p(w), _i64(T), k, H,
                                _p(out)), "combine")
    return out


def bf16_round_bits(v: np.ndarray) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_bf16_round_bits(_p(v), _i64(v.size), _p(out))
    return out


# ------------------------------------------------------- whole-layer helpers
def moe_layer(x, logits, k, weights, act, reps_budget=0, reps=None):
    """One full layer: route -> histogram -> replicas -> dispatch -> FFN (all rows) -> combine.
    Small shapes only (the FFN runs every row in plain C)."""
    T, E = logits.shape
    idx, w = route(logits, k)
    counts = histogram(idx, E)
    if reps is None and reps_budget > 0:
        reps = replicas(counts, T, k, reps_budget)
    d = dispatch(idx, E, reps)
    x_perm = permute(x, d["perm_src"])
    row_expert = np.repeat(np.arange(E, dtype=np.int32), np.diff(d["expert_off"]))
    y_perm = ffn_rows(x_perm, row_expert, *weights, act=act)
    out = combine(y_perm, d["inv_pos"], w)
    return dict(idx=idx, w=w, counts=counts, reps=reps, x_perm=x_perm, y_perm=y_perm, out=out, **d)


def token_forward(x_rows, idx, w, weights, act):
    """out[t] for a sample of tokens: x_rows [n,H], idx/w [n,k] -- each token's output
    depends only on its own row, so this is the layer output restricted to the sample.
    Returns (y [n,k,H] per-slot expert outputs, out [n,H])."""
    n, k = idx.shape
    xr = np.repeat(np.ascontiguousarray(x_rows), k, axis=0)
    y = ffn_rows(xr, idx.reshape(-1), *weights, act=act)
    inv = np.arange(n * k, dtype=np.int32).reshape(n, k)
    out = combine(y, inv, w)
    return y.reshape(n, k, -1), out
