"""Backward pass of one MoE layer -- TEST INFRASTRUCTURE ONLY.

The gradient, written out with the chain rule, of the forward the oracle
defines (moe_oracle.c): top-k softmax gate renormalised over the kept experts,
dispatch into expert-contiguous rows, expert FFN (SwiGLU or GELU), weighted
combine.  The backward pass is what the training-side pages run after the
forward they describe (PopFetcher wiki, method: the backward All-to-All; the
expert-load prediction study traces training iterations).

Plain numpy in float64, one expert at a time.  The pages say nothing about
precision in the backward pass; the reading taken extends the workloads'
"activations in the dtype, accumulation in fp32" to it: every tensor that is an
activation of the layer or the gradient of one is stored in the activation
dtype (rounded once, to nearest even), every product is accumulated exactly
(float64 here), d_h -- the inner product of one chain, consumed at once by
the activation gradient -- is never stored in the dtype, and the router-side
quantities dw and d_logits are float32, like the gate weights they differentiate:
  d_y   = w * d_out                  (one row per (token, slot)), rounded
  d_h   = d_y Wd                     (float64)
  SwiGLU: d_g = d_h * u * silu'(g), d_u = d_h * silu(g); GELU: d_z = d_h * gelu'(z)
                                     (from unrounded g, u, z), rounded
  d_xp  = d_g Wg + d_u Wu  (GELU: d_z W1), rounded
  d_x   = sum over the token's slots of d_xp, rounded
  d_Wd  = sum over the expert's rows of d_y^T h, rounded (h as the forward keeps it)
  d_Wg  = sum of d_g^T x_perm, d_Wu = sum of d_u^T x_perm (GELU: d_W1 = d_z^T x_perm), rounded
  dw[t,i] = <d_out[t], y_perm[row of (t,i)]>  (float64, y_perm as the forward keeps it)
  d_logits[t, e_j] = w_j (dw_j - sum_i w_i dw_i) for the kept experts, 0 elsewhere (float32)
The last line is the Jacobian of the softmax over the kept logits (renormalised
probabilities equal it); the other experts' logits do not reach the output.
It shares no code with the HIP library and never imports it.
"""
from __future__ import annotations

import math

import numpy as np

from . import bf16_round_bits, dispatch

_SQRT1_2 = 1.0 / math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _f64(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def _round(v: np.ndarray, bf16: bool) -> np.ndarray:
    """Round float64 values to the activation dtype (bf16 as bit patterns)."""
    return bf16_round_bits(v) if bf16 else np.asarray(v, dtype=np.float64).astype(np.float32)


def _erf(v: np.ndarray) -> np.ndarray:
    return np.vectorize(math.erf, otypes=[np.float64])(v)


def silu(g):
    return g / (1.0 + np.exp(-g))


def silu_grad(g):
    s = 1.0 / (1.0 + np.exp(-g))
    return s * (1.0 + g * (1.0 - s))


def gelu(z):
    return 0.5 * z * (1.0 + _erf(z * _SQRT1_2))


def gelu_grad(z):
    return 0.5 * (1.0 + _erf(z * _SQRT1_2)) + z * np.exp(-0.5 * z * z) * _INV_SQRT_2PI


def layer_backward(x, idx, w, weights, act, d_out):
    """Gradients of the layer output w.r.t. x, the router logits and the expert
    weights, given d_out = dL/d out.  x, d_out: [T, H] float32 or bf16 bits;
    idx, w: the routing ([T, k]); weights (w_gate [E,I,H], w_up [E,I,H] or None,
    w_down [E,H,I]) in the same dtype.  Returns a dict of rounded gradients
    (d_x, d_w_gate, d_w_up, d_w_down in the dtype, d_logits float32 [T, E]) and the
    float64 intermediates."""
    bf16 = np.asarray(x).dtype == np.uint16
    wg_, wu_, wd_ = weights
    Wg, Wd = _f64(wg_), _f64(wd_)
    Wu = None if wu_ is None else _f64(wu_)
    E, I, H = Wg.shape
    T, k = idx.shape
    X, dO = _f64(x), _f64(d_out)
    wt = np.asarray(w, dtype=np.float64)
    d = dispatch(idx, E)
    off, perm_src, inv = d["expert_off"], d["perm_src"], d["inv_pos"]
    M = T * k
    slot_w = np.empty(M)
    slot_w[inv.reshape(-1)] = wt.reshape(-1)
    Xp = X[perm_src]                                       # x_perm, exact
    dY = _f64(_round(slot_w[:, None] * dO[perm_src], bf16))  # d_y, rounded
    Yp = np.empty((M, H))
    dXp = np.empty((M, H))
    dWg = np.zeros((E, I, H))
    dWu = np.zeros((E, I, H)) if Wu is not None else None
    dWd = np.zeros((E, H, I))
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        xe = Xp[r0:r1]
        if Wu is not None:
            g, u = xe @ Wg[e].T, xe @ Wu[e].T
            h = _f64(_round(silu(g) * u, bf16))
        else:
            z = xe @ Wg[e].T
            h = _f64(_round(gelu(z), bf16))
        Yp[r0:r1] = _f64(_round(h @ Wd[e].T, bf16))
        dh = dY[r0:r1] @ Wd[e]
        if Wu is not None:
            dg = _f64(_round(dh * u * silu_grad(g), bf16))
            du = _f64(_round(dh * silu(g), bf16))
            dXp[r0:r1] = _f64(_round(dg @ Wg[e] + du @ Wu[e], bf16))
            dWg[e] = dg.T @ xe
            dWu[e] = du.T @ xe
        else:
            dz = _f64(_round(dh * gelu_grad(z), bf16))
            dXp[r0:r1] = _f64(_round(dz @ Wg[e], bf16))
            dWg[e] = dz.T @ xe
        dWd[e] = dY[r0:r1].T @ h
    dX = dXp[inv].sum(axis=1)                             # [T, H], slots summed in slot order
    dw = np.einsum("tih,th->ti", Yp[inv], dO)
    d_logits = np.zeros((T, E))
    s = (wt * dw).sum(axis=1, keepdims=True)
    np.put_along_axis(d_logits, idx.astype(np.int64), wt * (dw - s), axis=1)
    return dict(d_x=_round(dX, bf16), d_w_gate=_round(dWg, bf16),
                d_w_up=None if dWu is None else _round(dWu, bf16), d_w_down=_round(dWd, bf16),
                d_logits=d_logits.astype(np.float32), dw=dw, y_perm=Yp, d_y=dY, d_x_perm=dXp)


def sampled_backward(x, idx, w, weights, act, d_out, tokens, entries):
    """The same gradients as layer_backward, computed only where asked, for
    shapes too large to run whole: rows of d_x and d_logits for `tokens`, and
    weight-gradient entries `entries` = [(name, e, a, b)] with name in
    'd_w_gate', 'd_w_up', 'd_w_down' ([e][a, b] of that gradient).  Each value
    is formed by the definitions above from the rows that reach it (a token's
    own slots; all rows of expert e for a weight-gradient entry), in float64,
    with the same rounding points.  Returns (d_x [n, H], d_logits [n, E],
    {entry: value})."""
    bf16 = np.asarray(x).dtype == np.uint16
    wg_, wu_, wd_ = weights
    E, I, H = wg_.shape
    T, k = idx.shape
    dO = _f64(d_out)
    wt = np.asarray(w, dtype=np.float64)
    swiglu = wu_ is not None
    memo = {}   # per-expert columns shared by several entries (same values, computed once)
    rd = lambda v: _f64(_round(v, bf16))
    tokens = np.asarray(tokens)
    dX = np.zeros((len(tokens), H))
    dL = np.zeros((len(tokens), E))
    dw = np.zeros((len(tokens), k))
    vals = {}
    for e in range(E):
        sel = [(n, i) for n, t in enumerate(tokens) for i in range(k) if idx[t, i] == e]
        want = [en for en in entries if en[1] == e]
        if not sel and not want:
            continue
        Wg, Wd = _f64(wg_[e]), _f64(wd_[e])
        Wu = _f64(wu_[e]) if swiglu else None
        for n, i in sel:
            t = tokens[n]
            xr = _f64(x[t])
            g = Wg @ xr
            if swiglu:
                u = Wu @ xr
                h = rd(silu(g) * u)
            else:
                h = rd(gelu(g))
            dw[n, i] = rd(Wd @ h) @ dO[t]
            dy = rd(wt[t, i] * dO[t])
            dh = dy @ Wd
            if swiglu:
                dXp = rd(rd(dh * u * silu_grad(g)) @ Wg + rd(dh * silu(g)) @ Wu)
            else:
                dXp = rd(rd(dh * gelu_grad(g)) @ Wg)
            dX[n] += dXp
        if want:
            rows = np.argwhere(idx == e)                       # (t, i) of expert e's rows
            Xe = _f64(x[rows[:, 0]])
            dYe = rd(wt[rows[:, 0], rows[:, 1]][:, None] * dO[rows[:, 0]])
            for name, _, a, b in want:
                if name == "d_w_down":
                    if ("h", e, b) not in memo:
                        gb = Xe @ Wg[b]
                        memo[("h", e, b)] = rd(silu(gb) * (Xe @ Wu[b])) if swiglu else rd(gelu(gb))
                    v = dYe[:, a] @ memo[("h", e, b)]
                else:
                    if (name, e, a) not in memo:
                        ga = Xe @ Wg[a]
                        dha = dYe @ Wd[:, a]
                        if name == "d_w_gate" and swiglu:
                            memo[(name, e, a)] = rd(dha * (Xe @ Wu[a]) * silu_grad(ga))
                        elif name == "d_w_gate":
                            memo[(name, e, a)] = rd(dha * gelu_grad(ga))
                        else:
                            memo[(name, e, a)] = rd(dha * silu(ga))
                    v = memo[(name, e, a)] @ Xe[:, b]
                vals[(name, e, a, b)] = float(_f64(_round(np.array([v]), bf16))[0])
    s = (wt[tokens] * dw).sum(axis=1, keepdims=True)
    np.put_along_axis(dL, idx[tokens].astype(np.int64), wt[tokens] * (dw - s), axis=1)
    return _f64(_round(dX, bf16)), dL.astype(np.float32), vals
