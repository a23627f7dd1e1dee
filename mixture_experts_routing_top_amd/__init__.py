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

Every hot-path call takes `check`: an int32 device tensor of one element
(zeroed by the caller) that the kernels flag invalid input into;
moe_check_device_error(check) reads it back.  Output tensors passed in by the
caller are checked for shape, dtype and device before anything is launched.
"""
from __future__ import annotations

import ctypes

import torch

from ._native import LIB_PATH, MoEError, lib

__all__ = ["moe_route", "moe_stats_state_bytes", "moe_stats_init", "moe_stats", "moe_stats_load_state",
           "moe_plan_replicas",
           "moe_prediction_quality", "moe_dispatch_workspace_bytes",
           "moe_dispatch", "moe_expert_ffn_workspace_bytes", "moe_expert_ffn", "moe_combine", "moe_layer_forward",
           "moe_layer_forward_pipelined", "moe_backward_workspace_bytes", "moe_backward", "moe_check_device_error",
           "moe_expert_ffn_profiled", "new_check_word", "CHECK_BITS", "moe_dispatch_noalloc",
           "MoEError", "LIB_PATH", "MOE_F32", "MOE_BF16", "SWIGLU", "GELU", "GEMM_AUTO", "GEMM_GROUPED",
           "GEMM_DENSE", "GEMM_GROUPED_SMALL"]

MOE_F32, MOE_BF16 = 0, 1
SWIGLU, GELU = 0, 1
GEMM_AUTO, GEMM_GROUPED, GEMM_DENSE, GEMM_GROUPED_SMALL = 0, 1, 2, 3
_ACT = {"swiglu": SWIGLU, "gelu": GELU, SWIGLU: SWIGLU, GELU: GELU}
# bits of the device-check word (include/moe.h MOE_CHECK_*)
CHECK_BITS = {"logits": 1, "index": 2, "duplicate": 4, "counts": 8, "replicas": 16, "slots": 32, "rows": 64}
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


def _out(t, shape, dtype, dev, name):
    """A caller-supplied (or cached) output must match what the kernels will
    write: the same shape, dtype and device (the kernels bound-check only against
    the sizes taken from the inputs).  None: allocate one."""
    shape = tuple(int(v) for v in shape)
    if t is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if tuple(t.shape) != shape or t.dtype != dtype or t.device != torch.device(dev):
        raise ValueError(f"{name}: expected {dtype} {shape} on {dev}, got {t.dtype} {tuple(t.shape)} on {t.device}")
    return t


def _bytes_of(t, need, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.numel() * t.element_size() < need:
        have = t.numel() * t.element_size() if isinstance(t, torch.Tensor) else None
        raise ValueError(f"{name}: needs {need} bytes, got {have}")
    return t


def new_check_word(device="cuda"):
    """A zeroed device-check word (int32 [1]) for the `check` argument."""
    return torch.zeros(1, dtype=torch.int32, device=device)


def moe_check_device_error(check: torch.Tensor, stream=None) -> int:
    """Waits for the stream and reads the check word: returns 0 if nothing was
    flagged, else raises MoEError naming the flagged kinds (status -5)."""
    bits = ctypes.c_int32(0)
    rc = lib().moe_check_device_error(_ptr(check), ctypes.byref(bits), _stream(stream))
    if rc != 0:
        raise MoEError("moe_check_device_error", rc, lib().moe_last_error().decode(errors="replace"))
    return bits.value


# ------------------------------------------------------------------ routing
def moe_route(logits: torch.Tensor, k: int, topk_idx=None, topk_w=None, stream=None, check=None):
    T, E = logits.shape
    if logits.dtype != torch.float32:
        raise TypeError("router logits must be float32")
    dev = logits.device
    topk_idx = _out(topk_idx, (T, k), torch.int32, dev, "topk_idx")
    topk_w = _out(topk_w, (T, k), torch.float32, dev, "topk_w")
    _call("moe_route", _ptr(logits), ctypes.c_int64(T), E, k, _ptr(topk_idx), _ptr(topk_w), _ptr(check),
          _stream(stream))
    return topk_idx, topk_w


# --------------------------------------------------------------- statistics
def moe_stats_state_bytes(L: int, E: int, window: int) -> int:
    return int(lib().moe_stats_state_bytes(L, E, window))


def moe_stats_init(state: torch.Tensor, L: int, E: int, window: int, stream=None):
    _call("moe_stats_init", _ptr(state), ctypes.c_size_t(state.numel() * state.element_size()), L, E, window,
          _stream(stream))


def moe_stats(state: torch.Tensor, L: int, E: int, window: int, layer: int, it: int, topk_idx=None,
              prev_topk_idx=None, k: int = 0, counts=None, p_seq=None, cond=None, pred_next=None,
              replica_budget: int = 0, replicas=None, stream=None, check=None):
    """Outputs are optional (None: not written); those given must be int32/float32
    tensors of E (cond: E x E) elements."""
    T = 0 if topk_idx is None else topk_idx.shape[0]
    if topk_idx is not None:
        k = topk_idx.shape[1]
        if prev_topk_idx is not None and tuple(prev_topk_idx.shape) != tuple(topk_idx.shape):
            raise ValueError("prev_topk_idx must have the shape of topk_idx")
    dev = state.device
    for t, n, dt, name in ((counts, E, torch.int32, "counts"), (p_seq, E, torch.float32, "p_seq"),
                           (cond, E * E, torch.float32, "cond"), (pred_next, E, torch.float32, "pred_next"),
                           (replicas, E, torch.int32, "replicas")):
        if t is not None and (t.numel() != n or t.dtype != dt or t.device != dev):
            raise ValueError(f"{name}: expected {n} elements of {dt} on {dev}")
    _call("moe_stats", _ptr(state), ctypes.c_size_t(state.numel() * state.element_size()), L, E, window, layer,
          ctypes.c_int64(it), _ptr(topk_idx), _ptr(prev_topk_idx), ctypes.c_int64(T), k, _ptr(counts), _ptr(p_seq),
          _ptr(cond), _ptr(pred_next), replica_budget, _ptr(replicas), _ptr(check), _stream(stream))
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


def _dispatch_outputs(out, T, k, H, E, max_slots, dtype, dev, copy=True):
    o = dict(out or {})
    M = T * k
    for key, shape, dt in (("x_perm", (M, H), dtype), ("perm_src", (M,), torch.int32), ("inv_pos", (T, k), torch.int32),
                           ("expert_off", (E + 1,), torch.int32), ("slot_off", (max_slots + 1,), torch.int32),
                           ("slot_expert", (max_slots,), torch.int32), ("n_slots", (1,), torch.int32)):
        if key == "x_perm" and not copy:
            o[key] = None
            continue
        o[key] = _out(o.get(key), shape, dt, dev, key)
    return o


def moe_dispatch(x: torch.Tensor, topk_idx: torch.Tensor, E: int, replicas=None, max_slots=None, out=None,
                 workspace=None, stream=None, counts=None, check=None, replica_budget=0, copy=True):
    """counts (int32 [E], e.g. moe_stats' counts of this routing) is only compared
    with the routing when `check` is given.  replica_budget > 0 with replicas None:
    the dispatch plans the replicas from this routing's counts (max_slots defaults
    to E + replica_budget).  copy=False: no x_perm (None in the result); the FFN
    then gathers its rows from x with perm_src (moe_expert_ffn's row_src)."""
    T, H = x.shape
    if topk_idx.shape[0] != T or topk_idx.dtype != torch.int32:
        raise ValueError("topk_idx must be int32 [T, k] for the T rows of x")
    k = topk_idx.shape[1]
    dev = x.device
    max_slots = E + replica_budget if max_slots is None else max_slots
    for t, name in ((replicas, "replicas"), (counts, "counts")):
        if t is not None and (t.numel() != E or t.dtype != torch.int32):
            raise ValueError(f"{name} must be int32 [E]")
    o = _dispatch_outputs(out, T, k, H, E, max_slots, x.dtype, dev, copy)
    need = moe_dispatch_workspace_bytes(T, k, E)
    workspace = torch.empty(need, dtype=torch.uint8, device=dev) if workspace is None else \
        _bytes_of(workspace, need, "dispatch workspace")
    _call("moe_dispatch", _ptr(x), _dtype_code(x), ctypes.c_int64(T), H, _ptr(topk_idx), k, E, _ptr(counts),
          _ptr(replicas), replica_budget, max_slots, _ptr(o["x_perm"]), _ptr(o["perm_src"]), _ptr(o["inv_pos"]),
          _ptr(o["expert_off"]), _ptr(o["slot_off"]), _ptr(o["slot_expert"]), _ptr(o["n_slots"]), _ptr(workspace),
          ctypes.c_size_t(workspace.numel() * workspace.element_size()), _ptr(check), _stream(stream))
    return o


def moe_dispatch_noalloc(x: torch.Tensor, topk_idx: torch.Tensor, E: int, replicas=None, max_slots=None, out=None,
                         stream=None, counts=None, check=None, replica_budget=0):
    """moe_dispatch on the library's static device scratch (no workspace): for
    callers that cannot allocate.  `out` must hold every output (nothing is
    allocated here).  Calls that overlap on one GPU race."""
    T, H = x.shape
    if topk_idx.shape[0] != T or topk_idx.dtype != torch.int32:
        raise ValueError("topk_idx must be int32 [T, k] for the T rows of x")
    k = topk_idx.shape[1]
    max_slots = E + replica_budget if max_slots is None else max_slots
    need = ("x_perm", "perm_src", "inv_pos", "expert_off", "slot_off", "slot_expert", "n_slots")
    if out is None or any(key not in out for key in need):
        raise ValueError(f"moe_dispatch_noalloc allocates nothing: out must hold {need}")
    for t, name in ((replicas, "replicas"), (counts, "counts")):
        if t is not None and (t.numel() != E or t.dtype != torch.int32):
            raise ValueError(f"{name} must be int32 [E]")
    o = _dispatch_outputs(out, T, k, H, E, max_slots, x.dtype, x.device)
    _call("moe_dispatch_noalloc", _ptr(x), _dtype_code(x), ctypes.c_int64(T), H, _ptr(topk_idx), k, E, _ptr(counts),
          _ptr(replicas), replica_budget, max_slots, _ptr(o["x_perm"]), _ptr(o["perm_src"]), _ptr(o["inv_pos"]),
          _ptr(o["expert_off"]), _ptr(o["slot_off"]), _ptr(o["slot_expert"]), _ptr(o["n_slots"]), _ptr(check),
          _stream(stream))
    return o


# --------------------------------------------------------------- expert FFN
def moe_expert_ffn_workspace_bytes(dtype, M: int, H: int, I: int, max_slots: int) -> int:
    code = dtype if isinstance(dtype, int) else (MOE_BF16 if dtype == torch.bfloat16 else MOE_F32)
    return int(lib().moe_expert_ffn_workspace_bytes(code, ctypes.c_int64(M), H, I, max_slots))


def _ffn_args(x_perm, slot_off, slot_expert, n_slots, w_gate, w_up, w_down, y_perm, workspace, row_src=None):
    """row_src (int32 [M], e.g. moe_dispatch's perm_src): x_perm is then the token
    matrix x [T, H] and the FFN gathers row r from x_perm[row_src[r]]."""
    if row_src is not None:
        if row_src.dtype != torch.int32 or row_src.dim() != 1:
            raise ValueError("row_src must be int32 [M]")
        M, H = row_src.numel(), x_perm.shape[1]
    else:
        M, H = x_perm.shape
    E, I, H_ = w_gate.shape
    if H_ != H or tuple(w_down.shape) != (E, H, I) or (w_up is not None and tuple(w_up.shape) != (E, I, H)):
        raise ValueError("expert weights must be [E, I, H] (gate, up) and [E, H, I] (down) for x_perm's H")
    for w in (w_gate, w_up, w_down):
        if w is not None and w.dtype != x_perm.dtype:
            raise TypeError("expert weights must have the activation dtype")
    max_slots = slot_expert.numel()
    if slot_off.numel() != max_slots + 1 or n_slots.numel() != 1:
        raise ValueError("slot_off must hold max_slots + 1 entries and n_slots one")
    y_perm = _out(y_perm, (M, H), x_perm.dtype, x_perm.device, "y_perm")
    need = moe_expert_ffn_workspace_bytes(x_perm.dtype, M, H, I, max_slots)
    workspace = torch.empty(need, dtype=torch.uint8, device=x_perm.device) if workspace is None else \
        _bytes_of(workspace, need, "FFN workspace")
    return M, H, I, E, max_slots, y_perm, workspace


def moe_expert_ffn(x_perm: torch.Tensor, slot_off, slot_expert, n_slots, w_gate, w_up, w_down, act="swiglu",
                   path="grouped", y_perm=None, workspace=None, stream=None, check=None, row_src=None):
    """row_src: see _ffn_args (gathering the rows from x instead of x_perm)."""
    M, H, I, E, max_slots, y_perm, workspace = _ffn_args(x_perm, slot_off, slot_expert, n_slots, w_gate, w_up,
                                                         w_down, y_perm, workspace, row_src)
    _call("moe_expert_ffn", _ptr(x_perm), _ptr(row_src), ctypes.c_int64(x_perm.shape[0]), _dtype_code(x_perm),
          ctypes.c_int64(M), H, I, E, _ptr(slot_off),
          _ptr(slot_expert), _ptr(n_slots), max_slots, _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ACT[act],
          _PATH[path], _ptr(y_perm), _ptr(workspace), ctypes.c_size_t(workspace.numel() * workspace.element_size()),
          _ptr(check), _stream(stream))
    return y_perm


def moe_expert_ffn_profiled(x_perm: torch.Tensor, slot_off, slot_expert, n_slots, w_gate, w_up, w_down, events,
                            act="swiglu", path="grouped", y_perm=None, workspace=None, stream=None, check=None,
                            row_src=None):
    """moe_expert_ffn recording three torch.cuda.Event objects on the stream: before
    the gate/up GEMM, after it, after the down GEMM."""
    M, H, I, E, max_slots, y_perm, workspace = _ffn_args(x_perm, slot_off, slot_expert, n_slots, w_gate, w_up,
                                                         w_down, y_perm, workspace, row_src)
    for e in events:          # torch creates an event's handle on its first record
        if not e.cuda_event:
            e.record(stream if stream is not None else torch.cuda.current_stream())
    evs = (ctypes.c_void_p * 3)(*(e.cuda_event for e in events))
    _call("moe_expert_ffn_profiled", _ptr(x_perm), _ptr(row_src), ctypes.c_int64(x_perm.shape[0]),
          _dtype_code(x_perm), ctypes.c_int64(M), H, I, E, _ptr(slot_off),
          _ptr(slot_expert), _ptr(n_slots), max_slots, _ptr(w_gate), _ptr(w_up), _ptr(w_down), _ACT[act],
          _PATH[path], _ptr(y_perm), _ptr(workspace), ctypes.c_size_t(workspace.numel() * workspace.element_size()),
          _ptr(check), evs, _stream(stream))
    return y_perm


# ---------------------------------------------------------------- combine
def moe_combine(y_perm: torch.Tensor, inv_pos: torch.Tensor, topk_w: torch.Tensor, out=None, stream=None,
                check=None):
    M, H = y_perm.shape
    T, k = topk_w.shape
    if inv_pos.numel() != T * k or inv_pos.dtype != torch.int32 or topk_w.dtype != torch.float32:
        raise ValueError("inv_pos must be int32 [T, k] and topk_w float32 [T, k]")
    out = _out(out, (T, H), y_perm.dtype, y_perm.device, "out")
    _call("moe_combine", _ptr(y_perm), _dtype_code(y_perm), ctypes.c_int64(M), _ptr(inv_pos), _ptr(topk_w),
          ctypes.c_int64(T), k, H, _ptr(out), _ptr(check), _stream(stream))
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
    if M != T * k or tuple(y_perm.shape) != (M, H) or tuple(d_out.shape) != (T, H) or d_out.dtype != x_perm.dtype:
        raise ValueError("x_perm and y_perm must be [T*k, H] and d_out [T, H] of the activation dtype")
    o = dict(out or {})
    o["d_x"] = _out(o.get("d_x"), (T, H), x_perm.dtype, dev, "d_x")
    o["d_logits"] = _out(o.get("d_logits"), (T, E), torch.float32, dev, "d_logits")
    o["d_w_gate"] = _out(o.get("d_w_gate"), tuple(w_gate.shape), w_gate.dtype, dev, "d_w_gate")
    if w_up is not None:
        o["d_w_up"] = _out(o.get("d_w_up"), tuple(w_up.shape), w_up.dtype, dev, "d_w_up")
    o["d_w_down"] = _out(o.get("d_w_down"), tuple(w_down.shape), w_down.dtype, dev, "d_w_down")
    need = moe_backward_workspace_bytes(x_perm.dtype, T, k, H, I, E, act)
    workspace = torch.empty(need, dtype=torch.uint8, device=dev) if workspace is None else \
        _bytes_of(workspace, need, "backward workspace")
    _call("moe_backward", _ptr(x_perm), _ptr(y_perm), _dtype_code(x_perm), ctypes.c_int64(T), k, H, I, E,
          _ptr(topk_idx), _ptr(topk_w), _ptr(inv_pos), _ptr(expert_off), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
          _ACT[act], _ptr(d_out), _ptr(o["d_x"]), _ptr(o["d_logits"]), _ptr(o["d_w_gate"]), _ptr(o.get("d_w_up")),
          _ptr(o["d_w_down"]), _ptr(workspace), ctypes.c_size_t(workspace.numel() * workspace.element_size()),
          _stream(stream))
    return o


# ------------------------------------------------------ one layer, composed
def moe_layer_forward(x, logits, k, w_gate, w_up, w_down, act="swiglu", replica_budget=0, stats_state=None,
                      stats_dims=None, layer=0, it=0, prev_topk_idx=None, path="grouped", bufs=None, stream=None,
                      planned_replicas=None, check=None, ffn_events=None, copy_rows=False):
    """route -> stats -> dispatch -> FFN -> combine, all on `stream`.

    The dispatch writes the row map and the slot table but copies no rows: the
    FFN's gate/up GEMM gathers its rows from x through perm_src.  copy_rows=True
    runs the copying dispatch and hands the FFN x_perm (the result then holds
    x_perm, e.g. for moe_backward); both give bit-identical outputs.

    stats_state/stats_dims=(L, E, window) enable the windowed statistics
    (counts, p_seq, the conditional matrix, the prediction) and the replica
    plan from this iteration's counts, which the dispatch then takes.  Without
    statistics a replica budget is planned by the dispatch itself from the
    same counts (the same rule, so the same plan), and no moe_stats runs.
    planned_replicas (int32 [E], e.g. from moe_plan_replicas on the previous
    layer's prediction) replaces the count-based plan; it must hand out at
    most replica_budget copies.  `bufs` (a dict) caches outputs and
    workspaces between calls; they are reallocated when the shapes change.
    `check`: the device-check word passed to all five calls.  ffn_events:
    three torch.cuda.Event objects recorded around the two GEMM launches
    (moe_expert_ffn_profiled)."""
    T, E = logits.shape
    H = x.shape[1]
    I = w_gate.shape[1]
    dev = x.device
    max_slots = E + replica_budget
    b = bufs if bufs is not None else {}
    key = (T, k, E, H, I, max_slots, x.dtype, str(dev), copy_rows)
    if b.get("_key") != key:
        b.clear()
        b["_key"] = key
    idx, w = moe_route(logits, k, b.get("idx"), b.get("w"), stream, check)
    b["idx"], b["w"] = idx, w
    res = {"idx": idx, "w": w}
    replicas, counts = None, None
    if stats_state is not None:
        L_, E_, win = stats_dims
        for name, n, dt in (("counts", E, torch.int32), ("p_seq", E, torch.float32), ("replicas", E, torch.int32)):
            if name not in b:
                b[name] = torch.empty(n, dtype=dt, device=dev)
        if layer + 1 < L_:
            b.setdefault("cond", torch.empty((E, E), dtype=torch.float32, device=dev))
            b.setdefault("pred_next", torch.empty(E, dtype=torch.float32, device=dev))
        st = moe_stats(stats_state, L_, E_, win, layer, it, idx, prev_topk_idx, k, b["counts"], b["p_seq"],
                       b.get("cond") if layer + 1 < L_ else None, b.get("pred_next") if layer + 1 < L_ else None,
                       replica_budget, b["replicas"] if replica_budget > 0 and planned_replicas is None else None,
                       stream, check)
        res.update({kk: v for kk, v in st.items() if v is not None})
        replicas = b["replicas"] if replica_budget > 0 else None
        counts = b["counts"]
    if planned_replicas is not None:
        replicas = planned_replicas
        res["replicas"] = planned_replicas
    if "ws_d" not in b:
        b["ws_d"] = torch.empty(moe_dispatch_workspace_bytes(T, k, E), dtype=torch.uint8, device=dev)
    d = moe_dispatch(x, idx, E, replicas, max_slots, b.get("disp"), b["ws_d"], stream, counts, check,
                     replica_budget=replica_budget if replicas is None else 0, copy=copy_rows)
    b["disp"] = d
    if "y_perm" not in b:
        b["y_perm"] = torch.empty((T * k, H), dtype=x.dtype, device=dev)
    ffn_in, row_src = (d["x_perm"], None) if copy_rows else (x, d["perm_src"])
    if "ws_f" not in b:
        b["ws_f"] = torch.empty(moe_expert_ffn_workspace_bytes(x.dtype, T * k, H, I, max_slots), dtype=torch.uint8,
                                device=dev)
    if ffn_events is None:
        y = moe_expert_ffn(ffn_in, d["slot_off"], d["slot_expert"], d["n_slots"], w_gate, w_up, w_down, act,
                           path, b["y_perm"], b["ws_f"], stream, check, row_src=row_src)
    else:
        y = moe_expert_ffn_profiled(ffn_in, d["slot_off"], d["slot_expert"], d["n_slots"], w_gate, w_up, w_down,
                                    ffn_events, act, path, b["y_perm"], b["ws_f"], stream, check, row_src=row_src)
    out = moe_combine(y, d["inv_pos"], w, b.get("out"), stream, check)
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
    disp, done_d = {}, {}
    for c, t0, t1 in chunks:
        cb = b.setdefault(("chunk", c), {})
        if cb.get("_key") != (t1 - t0, k, E, H, x.dtype):   # per-chunk buffers keyed on the chunk's own T
            cb.clear()
            cb["_key"] = (t1 - t0, k, E, H, x.dtype)
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
