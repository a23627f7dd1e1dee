"""MI355X-native forward pass of one Mixture-of-Experts layer.

Thin Python binding over libmoe_mi355x.so (C ABI in include/moe.h).  These
functions only marshal arguments: they take torch tensors for device memory,
pass their pointers and the current HIP stream to the library, and allocate
outputs the caller did not supply.  Every step of the layer runs in the
library's HIP kernels; there is no fallback: if the library is missing or a
call fails, an exception is raised.

    idx, w = moe_route(logits, k)
    stats  = moe_stats(state, ...)          # counts, popularity, conditional, prediction, replicas
    plan   = moe_plan_replicas(pred_next, T*k, R)   # replicas for the next layer, ahead of its routing
    d      = moe_dispatch(x, idx, E, replicas, max_slots)
    y_perm = moe_expert_ffn(d["x_perm"], d["slot_off"], ..., w_gate, w_up, w_down)
    out    = moe_combine(y_perm, d["inv_pos"], w)
"""
from __future__ import annotations

import ctypes

import torch

from ._native import LIB_PATH, MoEError, lib

__all__ = ["moe_route", "moe_stats_state_bytes", "moe_stats_init", "moe_stats", "moe_stats_load_state",
           "moe_plan_replicas",
           "moe_prediction_quality", "moe_dispatch_workspace_bytes",
           "moe_dispatch", "moe_expert_ffn_workspace_bytes", "moe_expert_ffn", "moe_combine", "moe_layer_forward",
           "moe_layer_forward_pipelined", "moe_backward_workspace_bytes", "moe_backward",
           "MoEError", "LIB_PATH", "MOE_F32", "MOE_BF16", "SWIGLU", "GELU", "GEMM_AUTO", "GEMM_GROUPED",
           "GEMM_DENSE", "GEMM_GROUPED_SMALL"]

MOE_F32, MOE_BF16 = 0, 1
SWIGLU, GELU = 0, 1
GEMM_AUTO, GEMM_GROUPED, GEMM_DENSE, GEMM_GROUPED_SMALL = 0, 1, 2, 3
_ACT = {"swiglu": SWIGLU, "gelu": GELU, SWIGLU: SWIGLU, GELU: GELU}
_PATH = {"auto": GEMM_AUTO, "grouped": GEMM_GROUPED, "dense": GEMM_DENSE, "grouped_small": GEMM_GROUPED_SMALL,
         GEMM_AUTO: GEMM_AUTO, GEMM_GROUPED: GEMM_GROUPED, GEMM_DENSE: GEMM_DENSE,
         GEMM_GROUPED_SMALL: GEMM_GROUPED_SMALL}


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("tensors passed to the MoE library must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError(f"activations must be bfloat16 or float32, got {t.dtype}")


def _call(name, *args):
    rc = getattr(lib(), name)(*args)
    if rc != 0:
        raise MoEError(name, rc, lib().moe_last_error().decode(errors="replace"))


def _i32(n, dev):
    return torch.empty(n, dtype=torch.int32, device=dev)


# ------------------------------------------------------------------ routing
def moe_route(logits: torch.Tensor, k: int, topk_idx=None, topk_w=None, stream=None):
    T, E = logits.shape
    if logits.dtype != torch.float32:
        raise TypeError("router logits must be float32")
    dev = logits.device
    topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev) if topk_idx is None else topk_idx
    topk_w = torch.empty((T, k), dtype=torch.float32, device=dev) if topk_w is None else topk_w
    _call("moe_route", _ptr(logits), ctypes.c_int64(T), E, k, _ptr(topk_idx), _ptr(topk_w), _stream(stream))
    return topk_idx, topk_w


# --------------------------------------------------------------- statistics
def moe_stats_state_bytes(L: int, E: int, window: int) -> int:
    return int(lib().moe_stats_state_bytes(L, E, window))


def moe_stats_init(state: torch.Tensor, L: int, E: int, window: int, stream=None):
    _call("moe_stats_init", _ptr(state), ctypes.c_size_t(state.numel() * state.element_size()), L, E, window,
          _stream(stream))


def moe_stats(state: torch.Tensor, L: int, E: int, window: int, layer: int, it: int, topk_idx=None,
              prev_topk_idx=None, k: int = 0, counts=None, p_seq=None, cond=None, pred_next=None,
              replica_budget: int = 0, replicas=None, stream=None):
    T = 0 if topk_idx is None else topk_idx.shape[0]
    if topk_idx is not None:
        k = topk_idx.shape[1]
    _call("moe_stats", _ptr(state), ctypes.c_size_t(state.numel() * state.element_size()), L, E, window, layer,
          ctypes.c_int64(it), _ptr(topk_idx), _ptr(prev_topk_idx), ctypes.c_int64(T), k, _ptr(counts), _ptr(p_seq),
          _ptr(cond), _ptr(pred_next), replica_budget, _ptr(replicas), _stream(stream))
    return dict(counts=counts, p_seq=p_seq, cond=cond, pred_next=pred_next, replicas=replicas)


def moe_stats_load_state(state: torch.Tensor, L: int, E: int, window: int, layer: int, it: int, decay: float = 0.9,
                         p_decay=None, anomalous=None, summary=None, stream=None):
    """Decayed-window popularity, per-expert anomaly flags and [n_flagged, transient]
    of `layer` after iteration `it` was recorded."""
    dev = state.device
    p_decay = torch.empty(E, dtype=torch.float32, device=dev) if p_decay is None else p_decay
    anomalous = _i32(E, dev) if anomalous is None else anomalous
    summary = _i32(2, dev) if summary is None else summary
    _call("moe_stats_load_state", _ptr(state), ctypes.c_size_t(state.numel() * state.element_size()), L, E, window,
          layer, ctypes.c_int64(it), ctypes.c_double(decay), _ptr(p_decay), _ptr(anomalous), _ptr(summary),
          _stream(stream))
    return dict(p_decay=p_decay, anomalous=anomalous, summary=summary)


def moe_plan_replicas(pred: torch.Tensor, total: int, replica_budget: int, pred_counts=None, replicas=None,
                      stream=None):
    """Replica counts planned from a predicted distribution (e.g. moe_stats' pred_next)
    for a layer that will route `total` = T*k rows; returns (pred_counts, replicas)."""
    E = pred.numel()
    if pred.dtype != torch.float32:
        raise TypeError("the prediction must be float32")
    pred_counts = _i32(E, pred.device) if pred_counts is None else pred_counts
    replicas = _i32(E, pred.device) if replicas is None else replicas
    _call("moe_plan_replicas", _ptr(pred), E, ctypes.c_int64(total), replica_budget, _ptr(pred_counts),
          _ptr(replicas), _stream(stream))
    return pred_counts, replicas


def moe_prediction_quality(pred: torch.Tensor, counts: torch.Tensor, replicas=None, top_n: int = 5, out=None,
                           stream=None):
    """float32 [4] on the device: total-variation distance of the prediction to the
    actual shares, top-n hit rate, per-slot load std, max/mean slot load."""
    E = pred.numel()
    if pred.dtype != torch.float32 or counts.dtype != torch.int32:
        raise TypeError("pred must be float32 and counts int32")
    out = torch.empty(4, dtype=torch.float32, device=pred.device) if out is None else out
    _call("moe_prediction_quality", _ptr(pred), _ptr(counts), E, _ptr(replicas), top_n, _ptr(out), _stream(stream))
    return out


# ----------------------------------------------------------------- dispatch
def moe_dispatch_workspace_bytes(T: int, k: int, E: int) -> int:
    return int(lib().moe_dispatch_workspace_bytes(ctypes.c_int64(T), k, E))


def moe_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, E: int, replicas=None, max_slots=None, out=None,
                 workspace=None, stream=None):
    T, H = x.shape
    k = topk_idx.shape[1]
    M = T * k
    dev = x.device
    max_slots = E if max_slots is None else max_slots
    o = dict(out or {})
    o.setdefault("x_perm", torch.empty((M, H), dtype=x.dtype, device=dev))
    o.setdefault("perm_src", _i32(M, dev))
    o.setdefault("inv_pos", torch.empty((T, k), dtype=torch.int32, device=dev))
    o.setdefault("expert_off", _i32(E + 1, dev))
    o.setdefault("slot_off", _i32(max_slots + 1, dev))
    o.setdefault("slot_expert", _i32(max_slots, dev))
    o.setdefault("n_slots", _i32(1, dev))
    if workspace is None:
        workspace = torch.empty(moe_dispatch_workspace_bytes(T, k, E), dtype=torch.uint8, device=dev)
    _call("moe_dispatch", _ptr(x), _dtype_code(x), ctypes.c_int64(T), H, _ptr(topk_idx), k, E, _ptr(replicas),
          max_slots, _ptr(o["x_perm"]), _ptr(o["perm_src"]), _ptr(o["inv_pos"]), _ptr(o["expert_off"]),
          _ptr(o["slot_off"]), _ptr(o["slot_expert"]), _ptr(o["n_slots"]), _ptr(workspace),
          ctypes.c_size_t(workspace.numel()), _stream(stream))
    return o


# --------------------------------------------------------------- expert FFN
def moe_expert_ffn_workspace_bytes(dtype, M: int, H: int, I: int, max_slots: int) -> int:
    code = dtype if isinstance(dtype, int) else (MOE_BF16 if dtype == torch.bfloat16 else MOE_F32)
    return int(lib().moe_expert_ffn_workspace_bytes(code, ctypes.c_int64(M), H, I, max_slots))


def moe_expert_ffn(x_perm: torch.Tensor, slot_off, slot_expert, n_slots, w_gate, w_up, w_down, act="swiglu",
                   path="grouped", y_perm=None, workspace=None, stream=None):
    M, H = x_perm.shape
    E, I, _ = w_gate.shape
    max_slots = slot_expert.numel()
    y_perm = torch.empty_like(x_perm) if y_perm is None else y_perm
    if workspace is None:
        workspace = torch.empty(moe_expert_ffn_workspace_bytes(x_perm.dtype, M, H, I, max_slots), dtype=torch.uint8,
                                device=x_perm.device)
    _call("moe_expert_ffn", _ptr(x_perm), _dtype_code(x_perm), ctypes.c_int64(M), H, I, E, _ptr(slot_off),
          _ptr(slot_expert), _ptr(n_slots), max_slots, _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ACT[act],
          _PATH[path], _ptr(y_perm), _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(stream))
    return y_perm


# ---------------------------------------------------------------- combine
def moe_combine(y_perm: torch.Tensor, inv_pos: torch.Tensor, topk_w: torch.Tensor, out=None, stream=None):
    M, H = y_perm.shape
    T, k = topk_w.shape
    out = torch.empty((T, H), dtype=y_perm.dtype, device=y_perm.device) if out is None else out
    _call("moe_combine", _ptr(y_perm), _dtype_code(y_perm), ctypes.c_int64(M), _ptr(inv_pos), _ptr(topk_w),
          ctypes.c_int64(T), k, H, _ptr(out), _stream(stream))
    return out


# ----------------------------------------------------------------- backward
def moe_backward_workspace_bytes(dtype, T: int, k: int, H: int, I: int, E: int, act="swiglu") -> int:
    code = dtype if isinstance(dtype, int) else (MOE_BF16 if dtype == torch.bfloat16 else MOE_F32)
    return int(lib().moe_backward_workspace_bytes(code, ctypes.c_int64(T), k, H, I, E, _ACT[act]))


def moe_backward(x_perm, y_perm, topk_idx, topk_w, inv_pos, expert_off, w_gate, w_up, w_down, d_out, act="swiglu",
                 out=None, workspace=None, stream=None):
    """Gradients of the layer given d_out: dict(d_x, d_logits, d_w_gate, d_w_up, d_w_down).
    x_perm, inv_pos, expert_off from moe_dispatch; y_perm from moe_expert_ffn; the
    routing from moe_route."""
    T, k = topk_idx.shape
    M, H = x_perm.shape
    E, I, _ = w_gate.shape
    dev = x_perm.device
    o = dict(out or {})
    o.setdefault("d_x", torch.empty((T, H), dtype=x_perm.dtype, device=dev))
    o.setdefault("d_logits", torch.empty((T, E), dtype=torch.float32, device=dev))
    o.setdefault("d_w_gate", torch.empty_like(w_gate))
    if w_up is not None:
        o.setdefault("d_w_up", torch.empty_like(w_up))
    o.setdefault("d_w_down", torch.empty_like(w_down))
    if workspace is None:
        workspace = torch.empty(moe_backward_workspace_bytes(x_perm.dtype, T, k, H, I, E, act), dtype=torch.uint8,
                                device=dev)
    _call("moe_backward", _ptr(x_perm), _ptr(y_perm), _dtype_code(x_perm), ctypes.c_int64(T), k, H, I, E,
          _ptr(topk_idx), _ptr(topk_w), _ptr(inv_pos), _ptr(expert_off), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
          _ACT[act], _ptr(d_out), _ptr(o["d_x"]), _ptr(o["d_logits"]), _ptr(o["d_w_gate"]), _ptr(o.get("d_w_up")),
          _ptr(o["d_w_down"]), _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(stream))
    return o


# ------------------------------------------------------ one layer, composed
def moe_layer_forward(x, logits, k, w_gate, w_up, w_down, act="swiglu", replica_budget=0, stats_state=None,
                      stats_dims=None, layer=0, it=0, prev_topk_idx=None, path="grouped", bufs=None, stream=None,
                      planned_replicas=None):
    """route -> stats (+ replicas) -> dispatch -> FFN -> combine, all on `stream`.

    stats_state/stats_dims=(L, E, window) enable the windowed statistics; the
    replica budget needs this iteration's counts, which moe_stats produces.
    planned_replicas (int32 [E], e.g. from moe_plan_replicas on the previous
    layer's prediction) replaces that count-based plan; it must hand out at
    most replica_budget copies.  `bufs` (a dict) caches outputs and workspaces
    between calls."""
    T, E = logits.shape
    dev = x.device
    b = bufs if bufs is not None else {}
    idx, w = moe_route(logits, k, b.get("idx"), b.get("w"), stream)
    b["idx"], b["w"] = idx, w
    res = {"idx": idx, "w": w}
    replicas = None
    if stats_state is not None or replica_budget > 0:
        if stats_state is None:
            stats_dims = (1, E, 1)
            stats_state = b.get("_state")
            if stats_state is None:
                stats_state = torch.empty(moe_stats_state_bytes(*stats_dims), dtype=torch.uint8, device=dev)
                moe_stats_init(stats_state, *stats_dims, stream=stream)
                b["_state"] = stats_state
        L_, E_, win = stats_dims
        for key, n, dt in (("counts", E, torch.int32), ("p_seq", E, torch.float32), ("replicas", E, torch.int32)):
            if key not in b:
                b[key] = torch.empty(n, dtype=dt, device=dev)
        if layer + 1 < L_:
            b.setdefault("cond", torch.empty((E, E), dtype=torch.float32, device=dev))
            b.setdefault("pred_next", torch.empty(E, dtype=torch.float32, device=dev))
        st = moe_stats(stats_state, L_, E_, win, layer, it, idx, prev_topk_idx, k, b["counts"], b["p_seq"],
                       b.get("cond") if layer + 1 < L_ else None, b.get("pred_next") if layer + 1 < L_ else None,
                       replica_budget, b["replicas"] if replica_budget > 0 and planned_replicas is None else None,
                       stream)
        res.update({kk: v for kk, v in st.items() if v is not None})
        replicas = b["replicas"] if replica_budget > 0 else None
    if planned_replicas is not None:
        replicas = planned_replicas
        res["replicas"] = planned_replicas
    max_slots = E + replica_budget
    if "ws_d" not in b:
        b["ws_d"] = torch.empty(moe_dispatch_workspace_bytes(T, k, E), dtype=torch.uint8, device=dev)
    d = moe_dispatch(x, idx, E, replicas, max_slots, b.get("disp"), b["ws_d"], stream)
    b["disp"] = d
    if "y_perm" not in b:
        b["y_perm"] = torch.empty_like(d["x_perm"])
    if "ws_f" not in b:
        b["ws_f"] = torch.empty(moe_expert_ffn_workspace_bytes(x.dtype, T * k, x.shape[1], w_gate.shape[1], max_slots),
                                dtype=torch.uint8, device=dev)
    y = moe_expert_ffn(d["x_perm"], d["slot_off"], d["slot_expert"], d["n_slots"], w_gate, w_up, w_down, act, path,
                       b["y_perm"], b["ws_f"], stream)
    out = moe_combine(y, d["inv_pos"], w, b.get("out"), stream)
    b["out"] = out
    res.update(d)
    res.update(y_perm=y, out=out)
    return res


# ------------------------------------------- one layer, horizontally split
def moe_layer_forward_pipelined(x, logits, k, w_gate, w_up, w_down, act="swiglu", n_chunks=2, compute_stream=None,
                                memory_stream=None, bufs=None):
    """The layer split by rows into n_chunks token chunks, pipelined over two streams
    (EPS-MoE review, section 3: horizontal split of the input by rows, weights
    split by expert; the memory-bound kernels need few SMs and overlap the
    expert GEMMs).

    memory_stream: route, then every chunk's dispatch, then every chunk's
    combine (each waiting for its chunk's FFN); compute_stream: every chunk's
    expert FFN (each waiting for its dispatch).  Chunk c+1's dispatch can run
    while chunk c's GEMMs run, and chunk c's combine while chunk c+1's run.  The
    grouped GEMM path is used (no host readback), without replication; every
    output row depends only on its token, so the result equals
    moe_layer_forward's bit for bit.  The compute stream waits for the whole
    layer at the end; `bufs` caches the per-chunk buffers between calls."""
    T, E = logits.shape
    H = x.shape[1]
    I = w_gate.shape[1]
    dev = x.device
    cs = compute_stream if compute_stream is not None else torch.cuda.current_stream()
    ms = memory_stream if memory_stream is not None else cs
    b = bufs if bufs is not None else {}
    start = torch.cuda.Event()
    start.record(cs)
    ms.wait_event(start)
    idx, w = moe_route(logits, k, b.get("idx"), b.get("w"), ms)
    b["idx"], b["w"] = idx, w
    out = b.get("out")
    if out is None or out.shape != (T, H) or out.dtype != x.dtype:
        out = b["out"] = torch.empty((T, H), dtype=x.dtype, device=dev)
    bounds = [T * c // n_chunks for c in range(n_chunks + 1)]
    chunks = [(c, bounds[c], bounds[c + 1]) for c in range(n_chunks) if bounds[c + 1] > bounds[c]]
    t_max = max(t1 - t0 for _, t0, t1 in chunks) if chunks else 0
    if b.get("_ws_key") != (t_max, k, E, H, I, x.dtype):
        b["ws_d"] = torch.empty(moe_dispatch_workspace_bytes(t_max, k, E), dtype=torch.uint8, device=dev)
        b["ws_f"] = torch.empty(moe_expert_ffn_workspace_bytes(x.dtype, t_max * k, H, I, E), dtype=torch.uint8,
                                device=dev)
        b["_ws_key"] = (t_max, k, E, H, I, x.dtype)
        for c in range(n_chunks):
            b.pop(("chunk", c), None)
    disp, done_d = {}, {}
    for c, t0, t1 in chunks:
        cb = b.setdefault(("chunk", c), {})
        disp[c] = moe_dispatch(x[t0:t1], idx[t0:t1], E, None, E, cb.get("disp"), b["ws_d"], ms)
        cb["disp"] = disp[c]
        done_d[c] = torch.cuda.Event()
        done_d[c].record(ms)
    done_f = {}
    for c, t0, t1 in chunks:
        cb = b[("chunk", c)]
        d = disp[c]
        if "y_perm" not in cb or cb["y_perm"].shape != d["x_perm"].shape:
            cb["y_perm"] = torch.empty_like(d["x_perm"])
        cs.wait_event(done_d[c])
        moe_expert_ffn(d["x_perm"], d["slot_off"], d["slot_expert"], d["n_slots"], w_gate, w_up, w_down, act,
                       "grouped", cb["y_perm"], b["ws_f"], cs)
        done_f[c] = torch.cuda.Event()
        done_f[c].record(cs)
    for c, t0, t1 in chunks:
        ms.wait_event(done_f[c])
        moe_combine(b[("chunk", c)]["y_perm"], disp[c]["inv_pos"], w[t0:t1], out[t0:t1], ms)
    end = torch.cuda.Event()
    end.record(ms)
    cs.wait_event(end)
    return {"idx": idx, "w": w, "out": out}
