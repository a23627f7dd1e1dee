"""Throughput of one MoE layer's forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--replicas 8] [--no-cpu-baseline]

Workload: the Mixtral-8x7B-shaped layer (T=8192 tokens, H=4096, SwiGLU
I=14336, E=8 experts, top-2, bf16 activations and weights, fp32
accumulation), seeded synthetic inputs resident in HBM.  One step is one pass
of the whole hot path through the C ABI on one stream:

  moe_route -> moe_stats (counts, window popularity, co-occurrence with the
  previous layer's routing, conditional matrix, next-layer prediction,
  replica plan) -> moe_dispatch -> moe_expert_ffn -> moe_combine

The dispatch writes the row map (perm_src, inv_pos) and the slot table; the
FFN's gate/up GEMM gathers its rows from x through perm_src (no x_perm copy).

The timed layer is the middle layer of a three-layer statistics chain, so its
stats call exercises every statistic; the previous layer's routing is computed
once before timing.  Prints one JSON line: routed tokens/s (T / step time),
the roofline of the dominant kernel (the fused gate/up GEMM, timed with HIP
events on the library's stream), the layer's fraction of its roofline, and
the CPU oracle timed on a bounded sample on this host.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "routed tokens/s per MoE layer (Mixtral shape, T=8192) + % of roofline"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_gateup_mixtral_traffic.json")
GEMM_SOURCES = [os.path.join(ROOT, "mixture_experts_routing_top_amd", "csrc", f) for f in ("gemm.h", "ffn.hip")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--path", default="grouped", choices=["grouped", "grouped_small", "dense", "auto"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=12,
                    help="FFN rows each CPU-baseline process runs (sample)")
    ap.add_argument("--crossover", action="store_true",
                    help="time the grouped and the dense expert-FFN paths on the DeepSeek-V2 T sweep and on the "
                         "GEMM shapes profiled by EPS-MoE, print one JSON line per case, and exit")
    ap.add_argument("--cases", default="",
                    help="with --crossover: comma-separated case labels to run (e.g. dsv2_T4096); default all")
    ap.add_argument("--paths", default="grouped,grouped_small,dense,auto",
                    help="with --crossover: comma-separated tilings to time")
    ap.add_argument("--configs", action="store_true",
                    help="routed tokens/s and roofline fraction of every workload (one line each)")
    ap.add_argument("--stats", action="store_true",
                    help="time moe_stats with co-occurrence (a chained layer) on the workloads' shapes")
    ap.add_argument("--backward", action="store_true",
                    help="time the layer's backward pass (moe_backward) on the Mixtral layer")
    ap.add_argument("--pipeline", action="store_true",
                    help="horizontal-split pipeline and memory kernels on CU-masked streams (Mixtral layer)")
    ap.add_argument("--predict", action="store_true",
                    help="score the next-layer prediction and the replica plans on the 12-layer chain")
    ap.add_argument("--vs-hipblaslt", action="store_true",
                    help="dense single-expert gate/up and down GEMMs of the Mixtral shape next to hipBLASLt "
                         "(torch.matmul) on the same shapes, in one process")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy a 256 MiB buffer 3 times (reference for the HBM byte counters) and exit")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """Hash of the code the gate/up GEMM is built from (the kernel template and its
    launcher), comments and whitespace removed: comment edits keep the counters valid."""
    import re
    h = hashlib.sha256()
    for path in GEMM_SOURCES:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(flop_unit_rows: int):
    """HBM bytes per gate/up launch from the committed rocprofv3 PMC runs, only if
    they were taken on the current kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    rec = json.load(open(TRAFFIC_FILE))
    if rec.get("gemm_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def memory_phase_bytes(T, H, E, k, s=2, copy_rows=False):
    """Algorithmic bytes of the memory-bound phases: route (logits in, idx + w
    out), dispatch (idx in, perm_src + inv_pos out; with copy_rows also x in and
    x_perm out, the rows the gathering FFN otherwise reads from x itself) and
    combine (y_perm in, out, inv_pos + w)."""
    M = T * k
    return (T * E * 4 + T * k * 8
            + T * k * 4 + M * 8 + ((T * H * s + M * H * s) if copy_rows else 0)
            + M * H * s + T * H * s + M * 8)


def algorithmic_layer_work(T, H, I, E, k, n_mat):
    """Algorithmic flops and HBM bytes of one layer (intermediates and padding excluded)."""
    M = T * k
    flops = 2.0 * M * H * I * n_mat
    s = 2
    w_bytes = E * n_mat * H * I * s
    mem = memory_phase_bytes(T, H, E, k, s)
    return flops, w_bytes, mem


class TimingEvent:
    """A HIP event for timestamps inside a step: created with
    hipEventDisableSystemFence, so recording it between two kernels does not
    write back and invalidate the caches as a default event does (about 6 us
    per record here, and the next kernel starts on emptied caches).  Its times
    are read only after a device synchronize.  Same interface as
    torch.cuda.Event where bench.py and moe_expert_ffn_profiled use one."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        if TimingEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")   # the HIP runtime torch has loaded
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            TimingEvent._hip = hip
        self.h = ctypes.c_void_p()
        rc = self._hip.hipEventCreateWithFlags(ctypes.byref(self.h), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")

    @property
    def cuda_event(self):
        return self.h.value

    def record(self, stream):
        rc = self._hip.hipEventRecord(self.h, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_time(self, other):
        ms = ctypes.c_float()
        rc = self._hip.hipEventElapsedTime(ctypes.byref(ms), self.h, other.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def __del__(self):
        if self.h.value and TimingEvent._hip is not None:
            TimingEvent._hip.hipEventDestroy(self.h)


def spin_cycles(torch, stream, ms):
    """Argument of torch.cuda._sleep that keeps the GPU busy for about `ms`
    milliseconds (its counter's rate differs between devices: measured here)."""
    n = 1 << 20
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(1024)  # the first launch loads the kernel: keep it out of the timing
    torch.cuda.synchronize()
    a.record(stream)
    torch.cuda._sleep(n)
    b.record(stream)
    torch.cuda.synchronize()
    return max(1, int(n * ms / max(a.elapsed_time(b), 1e-3)))


def memory_phase_summary(T, H, E, k, warm, cold):
    """Routing, dispatch and combine against HBM: their algorithmic bytes
    (memory_phase_bytes: the layer's dispatch copies no rows, the FFN gathers
    them from x) over their event-timed GPU phase times (which also hold the
    GPU's gaps between launches)."""
    b = memory_phase_bytes(T, H, E, k)
    M = T * k
    # the same bytes per phase (route; dispatch's index arrays; combine's rows)
    per = {"route": T * E * 4 + T * k * 8, "dispatch": T * k * 4 + M * 8, "combine": M * H * 2 + T * H * 2 + M * 8}
    assert sum(per.values()) == b
    out = {"bytes": b}
    for label, ph in (("warm", warm), ("cold", cold)):
        us = ph["route"] + ph["dispatch"] + ph["combine"]
        out[label] = {"us": round(us, 2), "GBps": round(b / (us * 1e-6) / 1e9, 1),
                      "frac_of_hbm": round(b / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 3),
                      "per_phase": {n: {"bytes": per[n], "us": ph[n],
                                        "frac_of_hbm": round(per[n] / (ph[n] * 1e-6) / 1e9 / PEAK_HBM_GBS, 3)}
                                    for n in per}}
    return out


_CPU = {}   # inputs of the CPU baseline's FFN workers (inherited by the forked processes)


def _cpu_ffn_worker(span):
    """One process of the N-core leg: the oracle's FFN (plain single-threaded C)
    on its own disjoint run of the sampled rows."""
    import oracle
    lo, hi = span
    sel = _CPU["sel"][lo:hi]
    t0 = time.perf_counter()
    oracle.ffn_rows(_CPU["x_perm"][sel], _CPU["expert"][sel], *_CPU["wts"], act=_CPU["act"])
    return time.perf_counter() - t0


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, x, logits, wts, prev_logits, R, rows_per_proc):
    """The oracle on this host, on a bounded sample of the same workload.

    One core: routing, window statistics, replicas, dispatch/permute and combine
    at full size (the oracle is single-threaded).  N cores: the expert FFN -- the
    same single-threaded oracle code -- in N processes over disjoint runs of
    rows (rows are independent after dispatch), each process `rows_per_proc`
    rows of an even sample of the T*k rows; its wall time is extrapolated to all
    rows.  Must run before the GPU is touched (the workers are forked)."""
    import multiprocessing

    import numpy as np

    import oracle

    T, E, k = cfg.T, cfg.E, cfg.k
    t0 = time.perf_counter()
    prev_idx, _ = oracle.route(prev_logits, k)
    idx, w = oracle.route(logits, k)
    st = oracle.WindowStats(3, E, 10)
    st.record(0, 0, prev_idx)
    counts = st.record(1, 0, idx, prev_idx)
    st.outputs(1)
    reps = oracle.replicas(counts, T, k, R) if R else None
    d = oracle.dispatch(idx, E, reps)
    x_perm = oracle.permute(x, d["perm_src"])
    t_mem = time.perf_counter() - t0
    y_fake = np.zeros_like(x_perm)       # combine's cost does not depend on the values
    t2 = time.perf_counter()
    oracle.combine(y_fake, d["inv_pos"], w)
    t_comb = time.perf_counter() - t2
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    n_proc = max(1, min(16, affinity))
    n_rows = n_proc * rows_per_proc
    _CPU.update(x_perm=x_perm, expert=np.repeat(np.arange(E, dtype=np.int32), np.diff(d["expert_off"])),
                sel=np.linspace(0, T * k - 1, n_rows).astype(np.int64), wts=wts, act=cfg.act)
    oracle.lib()                          # built and loaded once, before the fork
    with multiprocessing.get_context("fork").Pool(n_proc) as pool:
        pool.map(len, [()] * n_proc)      # workers up before timing
        t1 = time.perf_counter()
        per_proc = pool.map(_cpu_ffn_worker, [(i * rows_per_proc, (i + 1) * rows_per_proc) for i in range(n_proc)])
        wall_ffn = time.perf_counter() - t1
    _CPU.clear()
    t_ffn_n = wall_ffn * (T * k) / n_rows                     # all rows on n_proc cores
    t_ffn_1 = float(np.mean(per_proc)) / rows_per_proc * (T * k)  # all rows on one core
    total_n = t_mem + t_comb + t_ffn_n
    total_1 = t_mem + t_comb + t_ffn_1
    return {"value": round(T / total_n, 3), "unit": "tokens/s", "cores": n_proc, "kind": "oracle",
            "one_core_value": round(T / total_1, 3),
            "n_core_wall_s": round(total_n, 1), "one_core_wall_s": round(total_1, 1),
            "host": {"nproc": os.cpu_count(), "affinity_cpus": affinity, "cpu_model": cpu_model()},
            "sample": (f"routing, window statistics, replicas, dispatch and combine at full size (T={T}) on one "
                       f"core ({t_mem + t_comb:.1f} s); expert FFN on {n_rows} of {T * k} rows, {rows_per_proc} "
                       f"per process in {n_proc} processes ({wall_ffn:.1f} s wall, "
                       f"{float(np.sum(per_proc)):.1f} s CPU), extrapolated to all rows")}


def crossover(moe, synth, torch, np, cases=(), paths=("grouped", "grouped_small", "dense", "auto")):
    """Grouped (256-row tiles) vs dense padded (64-row tiles) expert FFN.  Routing
    and slot tables come from the seeded generators; weights and activations are
    random device tensors (values do not change the timing).  `cases` limits the
    run to those case labels (all when empty), `paths` to those tilings."""
    dev = torch.device("cuda:0")
    torch.manual_seed(0)

    def wanted(label):
        return not cases or label in cases

    def time_paths(x_perm, slot_off, slot_expert, n_slots, wg, wu, wd, label, extra):
        if not wanted(label):
            return
        M, H = x_perm.shape
        I = wg.shape[1]
        ws = torch.empty(moe.moe_expert_ffn_workspace_bytes(x_perm.dtype, M, H, I, slot_expert.numel()),
                         dtype=torch.uint8, device=dev)
        y = torch.empty_like(x_perm)
        res = dict(case=label, **extra)
        offs = slot_off.cpu().numpy()[: int(n_slots.item()) + 1].astype(np.int64)
        rows = np.diff(offs)
        # the grouped tiling: 256-row tiles, a range of <= 64 rows as one 64-row tile
        short = (rows > 0) & (rows <= 64)
        res["tiles"] = {"g256": int(np.sum(np.where(short, 0, (rows + 255) // 256))),
                        "g256_short64": int(np.count_nonzero(short)), "g64": int(np.sum((rows + 63) // 64)),
                        "d64": int(np.count_nonzero(rows) * ((rows.max() + 63) // 64))}
        for path in paths:
            for _ in range(2):
                moe.moe_expert_ffn(x_perm, slot_off, slot_expert, n_slots, wg, wu, wd, "swiglu", path, y, ws)
            torch.cuda.synchronize()
            ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(5)]
            for i in range(5):
                moe.moe_expert_ffn_profiled(x_perm, slot_off, slot_expert, n_slots, wg, wu, wd, ev[i], "swiglu", path,
                                            y, ws)
            torch.cuda.synchronize()
            g = float(np.median([ev[i][0].elapsed_time(ev[i][1]) for i in range(5)]))
            d = float(np.median([ev[i][1].elapsed_time(ev[i][2]) for i in range(5)]))
            res[path] = {"gateup_ms": round(g, 4), "down_ms": round(d, 4), "ffn_ms": round(g + d, 4)}
        # which path AUTO takes (it reads the slot sizes back): compare its output timing-free
        fixed = [p for p in ("grouped", "grouped_small", "dense") if p in res]
        if fixed:
            res["fastest"] = min(fixed, key=lambda p: res[p]["ffn_ms"])
        print(json.dumps(res), flush=True)

    cfg0 = synth.CONFIGS["dsv2"]
    E, H, I, k = cfg0.E, cfg0.H, cfg0.I, cfg0.k
    wg = (torch.randn(E, I, H, device=dev) * H ** -0.5).to(torch.bfloat16)
    wu = (torch.randn(E, I, H, device=dev) * H ** -0.5).to(torch.bfloat16)
    wd = (torch.randn(E, H, I, device=dev) * I ** -0.5).to(torch.bfloat16)
    for T in synth.DSV2_T_SWEEP:
        if not wanted(f"dsv2_T{T}"):
            continue
        cfg = cfg0.with_T(T)
        idx, _ = moe.moe_route(torch.from_numpy(synth.logits(cfg, 0, 0)).to(dev), k)
        x = torch.randn(T, H, device=dev).to(torch.bfloat16)
        d = moe.moe_dispatch(x, idx, E, None, E)
        counts = np.diff(d["expert_off"].cpu().numpy())
        time_paths(d["x_perm"], d["slot_off"], d["slot_expert"], d["n_slots"], wg, wu, wd, f"dsv2_T{T}",
                   {"E": E, "k": k, "H": H, "I": I, "rows": int(T * k), "max_rows": int(counts.max()),
                    "mean_rows": round(float(counts.mean()), 1), "empty_experts": int((counts == 0).sum())})
    del wg, wu, wd
    # coarse-grained layers: Mixtral- and DBRX-shaped routing (large per-expert counts)
    for name in ("mixtral", "dbrx"):
        cfg = synth.CONFIGS[name]
        if not any(wanted(f"{name}_T{T}") for T in (cfg.T // 8, cfg.T)):
            continue
        E, H, I, k = cfg.E, cfg.H, cfg.I, cfg.k
        wg = (torch.randn(E, I, H, device=dev) * H ** -0.5).to(torch.bfloat16)
        wu = (torch.randn(E, I, H, device=dev) * H ** -0.5).to(torch.bfloat16)
        wd = (torch.randn(E, H, I, device=dev) * I ** -0.5).to(torch.bfloat16)
        for T in (cfg.T // 8, cfg.T):
            if not wanted(f"{name}_T{T}"):
                continue
            c = cfg.with_T(T)
            idx, _ = moe.moe_route(torch.from_numpy(synth.logits(c, 0, 0)).to(dev), k)
            x = torch.randn(T, H, device=dev).to(torch.bfloat16)
            d = moe.moe_dispatch(x, idx, E, None, E)
            counts = np.diff(d["expert_off"].cpu().numpy())
            time_paths(d["x_perm"], d["slot_off"], d["slot_expert"], d["n_slots"], wg, wu, wd, f"{name}_T{T}",
                       {"E": E, "k": k, "H": H, "I": I, "rows": int(T * k), "max_rows": int(counts.max()),
                        "mean_rows": round(float(counts.mean()), 1)})
        del wg, wu, wd
    # single-expert GEMM shapes M x K x N printed by EPS-MoE (K = H; N = I of one projection)
    for M, K_, N_ in ((512, 5120, 1536), (2048, 5120, 1536), (512, 5120, 14336)):
        if not wanted(f"gemm_{M}x{K_}x{N_}"):
            continue
        x = torch.randn(M, K_, device=dev).to(torch.bfloat16)
        g1 = (torch.randn(1, N_, K_, device=dev) * K_ ** -0.5).to(torch.bfloat16)
        u1 = (torch.randn(1, N_, K_, device=dev) * K_ ** -0.5).to(torch.bfloat16)
        d1 = (torch.randn(1, K_, N_, device=dev) * N_ ** -0.5).to(torch.bfloat16)
        so = torch.tensor([0, M], dtype=torch.int32, device=dev)
        se = torch.zeros(1, dtype=torch.int32, device=dev)
        ns = torch.ones(1, dtype=torch.int32, device=dev)
        time_paths(x, so, se, ns, g1, u1, d1, f"gemm_{M}x{K_}x{N_}", {"M": M, "K": K_, "N": N_})


def predict_quality(moe, synth, torch, np, name="popfetcher", R=8, iters=None):
    """Prediction quality and load balance on a chained workload, all on the GPU.

    Per iteration and layer l >= 1: layer l-1's statistics predict layer l's
    popularity (moe_stats pred_next); moe_plan_replicas plans R copies from it
    before layer l routes; after routing, moe_prediction_quality scores the
    prediction and three plans against the actual counts: no replicas, the
    predicted plan, and the plan from the actual counts (moe_stats replicas)."""
    cfg = synth.CONFIGS[name]
    L, E, k, win, T = cfg.L, cfg.E, cfg.k, cfg.window, cfg.T
    iters = cfg.iters if iters is None else iters
    dev = torch.device("cuda:0")
    state = torch.empty(moe.moe_stats_state_bytes(L, E, win), dtype=torch.uint8, device=dev)
    moe.moe_stats_init(state, L, E, win)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    pred = torch.empty(E, dtype=torch.float32, device=dev)
    reps_now = torch.empty(E, dtype=torch.int32, device=dev)
    rows = []
    plan_ev, qual_ev = [], []
    for it in range(iters):
        prev_idx, plan, pred_prev = None, None, None
        top1 = None
        for layer in range(L):
            lg = synth.logits(cfg, layer, it, top1)
            idx, _ = moe.moe_route(torch.from_numpy(lg).to(dev), k)
            last = layer + 1 >= L
            moe.moe_stats(state, L, E, win, layer, it, idx, prev_idx, k, counts, None, None,
                          None if last else pred, R, reps_now)
            if plan is not None:
                q = [moe.moe_prediction_quality(pred_prev, counts, r, 5) for r in (None, plan, reps_now)]
                rows.append((it, layer, torch.stack(q).cpu().numpy()))
            if not last:
                pred_prev = pred.clone()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                _, plan = moe.moe_plan_replicas(pred_prev, T * k, R)
                e1.record()
                plan_ev.append((e0, e1))
                q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                q0.record()
                moe.moe_prediction_quality(pred_prev, counts, plan, 5)
                q1.record()
                qual_ev.append((q0, q1))
            top1 = idx[:, 0].cpu().numpy()
            prev_idx = idx
    torch.cuda.synchronize()

    def summary(sel):
        a = np.stack([r[2] for r in rows if sel(r)])  # [n, 3 plans, 4 measures]
        return {"samples": int(a.shape[0]),
                "tv_distance_mean": round(float(a[:, 1, 0].mean()), 5),
                "top5_hit_mean": round(float(a[:, 1, 1].mean()), 4),
                "slot_load_std": {"none": round(float(a[:, 0, 2].mean()), 1),
                                  "predicted_plan": round(float(a[:, 1, 2].mean()), 1),
                                  "counts_plan": round(float(a[:, 2, 2].mean()), 1)},
                "max_over_mean_load": {"none": round(float(a[:, 0, 3].mean()), 3),
                                       "predicted_plan": round(float(a[:, 1, 3].mean()), 3),
                                       "counts_plan": round(float(a[:, 2, 3].mean()), 3)}}

    return {"prediction": {
        "workload": f"{name}-shaped chain: L={L} E={E} k={k} T={T} window={win} iterations={iters} "
                    f"gamma={cfg.gamma} c={cfg.c}",
        "replica_budget": R,
        "all_layers_iterations": summary(lambda r: True),
        "after_first_iteration": summary(lambda r: r[0] >= 1),
        "plan_kernel_us": round(float(np.median([a.elapsed_time(b) for a, b in plan_ev])) * 1e3, 2),
        "quality_kernel_us": round(float(np.median([a.elapsed_time(b) for a, b in qual_ev])) * 1e3, 2)}}


def cu_masked_stream(torch, n_cu, total):
    """A stream limited to n_cu compute units, spread evenly over the 8 XCDs under
    either CU numbering (XCD-major or XCD-interleaved bits); None if refused."""
    words = [0] * (total // 32)
    per = n_cu // 8
    if n_cu >= total:
        words = [0xFFFFFFFF] * (total // 32)
    else:
        for x in range(8):
            for m in range(per):
                words[x] |= 1 << ((x + 8 * m) % 32 if per <= 4 else m)
    hip = ctypes.CDLL("libamdhip64.so")
    arr = (ctypes.c_uint32 * len(words))(*words)
    handle = ctypes.c_void_p()
    if hip.hipExtStreamCreateWithCUMask(ctypes.byref(handle), ctypes.c_uint32(len(words)), arr) != 0:
        return None, None
    return torch.cuda.ExternalStream(handle.value), (hip, handle)


def pipeline_bench(moe, synth, torch, np, steps=10, warmup=3):
    """EPS-MoE's horizontal split on one GPU: the Mixtral layer unsplit versus split
    into n chunks over a compute and a memory stream; and the memory-bound kernels
    alone on streams limited to n CUs (do they, like communication kernels, need
    only a few?).  No replication, grouped GEMM path."""
    cfg = synth.CONFIGS["mixtral"]
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    dev = torch.device("cuda:0")

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    wg, wu, wd = (dev_bf16(w) for w in synth.expert_weights(cfg, threads=16))
    x = dev_bf16(synth.hidden0(cfg, 0))
    logits = torch.from_numpy(synth.logits(cfg, 0, 0)).to(dev)
    cs = torch.cuda.current_stream()

    def timed(fn, stream):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    res = {"workload": f"Mixtral-shaped layer T={T} H={H} I={I} E={E} k={k} bf16, no replication"}
    bufs = {}
    ref = None
    base = timed(lambda: moe.moe_layer_forward(x, logits, k, wg, wu, wd, "swiglu", 0, bufs=bufs, stream=cs), cs)
    ref = bufs["out"].clone()
    res["unsplit_ms"] = round(base, 4)
    total_cu = torch.cuda.get_device_properties(0).multi_processor_count
    ms = torch.cuda.Stream()
    split = {}
    for n in (1, 2, 4, 8):
        pb = {}
        t = timed(lambda: moe.moe_layer_forward_pipelined(x, logits, k, wg, wu, wd, "swiglu", n, cs, ms, pb), cs)
        split[n] = {"ms": round(t, 4), "speedup": round(base / t, 4), "bit_identical": bool(torch.equal(pb["out"], ref))}
    res["split_two_streams"] = split
    sweep, handles = {}, []
    d = moe.moe_dispatch(x, bufs["idx"], E, None, E)
    y = d["x_perm"]
    ws = torch.empty(moe.moe_dispatch_workspace_bytes(T, k, E), dtype=torch.uint8, device=dev)
    out = torch.empty_like(x)
    row_bytes = (k + 1) * T * H * 2   # permute: x + x_perm; combine: y_perm + out
    for n_cu in (8, 16, 32, 64, 128, total_cu):
        st, h = cu_masked_stream(torch, n_cu, total_cu)
        if st is None:
            sweep[n_cu] = "stream creation refused"
            continue
        handles.append(h)
        td = timed(lambda: moe.moe_dispatch(x, bufs["idx"], E, None, E, d, ws, st), st)
        tc = timed(lambda: moe.moe_combine(y, d["inv_pos"], bufs["w"], out, st), st)
        sweep[n_cu] = {"dispatch_us": round(td * 1e3, 1), "combine_us": round(tc * 1e3, 1),
                       "dispatch_TBps": round(row_bytes / (td * 1e-3) / 1e12, 2),
                       "combine_TBps": round(row_bytes / (tc * 1e-3) / 1e12, 2)}
        if n_cu in (32, 64):
            pb = {}
            t = timed(lambda: moe.moe_layer_forward_pipelined(x, logits, k, wg, wu, wd, "swiglu", 4, cs, st, pb), cs)
            sweep[n_cu]["split4_memory_stream_ms"] = round(t, 4)
            sweep[n_cu]["split4_bit_identical"] = bool(torch.equal(pb["out"], ref))
    torch.cuda.synchronize()
    for hip, h in handles:
        hip.hipStreamDestroy(h)
    res["memory_kernels_on_n_cus"] = sweep
    return {"pipeline": res}


PEAK_FP32_TFLOPS = 157.3         # MI355X dense fp32 MFMA


def configs_bench(moe, synth, torch, np, steps=20, warmup=20):
    """Every workload's layer forward on the GPU: routed tokens/s per layer and the
    fraction of its roofline, t_roof = max(flop / MFMA peak, active expert weights /
    HBM) + memory-phase bytes / HBM (routing, dispatch, combine; algorithmic)."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def to_dev(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    def roofline(cfg, counts):
        s = cfg.elem_bytes
        flop = 2.0 * cfg.T * cfg.k * cfg.H * cfg.I * cfg.n_mat
        active = int(np.count_nonzero(counts))
        w_bytes = active * cfg.n_mat * cfg.I * cfg.H * s
        mem = memory_phase_bytes(cfg.T, cfg.H, cfg.E, cfg.k, s)
        peak = (PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS) * 1e12
        t = max(flop / peak, w_bytes / (PEAK_HBM_GBS * 1e9)) + mem / (PEAK_HBM_GBS * 1e9)
        bound = "mfma" if flop / peak >= w_bytes / (PEAK_HBM_GBS * 1e9) else "hbm (weight streaming)"
        return t, bound

    def report(name, cfg, ms, counts, extra):
        t_roof, bound = roofline(cfg, counts)
        rec = {"workload": name, "T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "k": cfg.k, "act": cfg.act,
               "dtype": cfg.dtype, "ms_per_layer": round(ms, 4),
               "routed_tokens_per_s_per_layer": round(cfg.T / (ms * 1e-3), 1),
               "roofline_ms": round(t_roof * 1e3, 4), "roofline_frac": round(t_roof / (ms * 1e-3), 4),
               "roofline_bound": bound}
        rec.update(extra)
        print(json.dumps({"config": rec}), flush=True)

    cache = {}

    def weights_of(cfg):
        # weights do not depend on T: one upload per workload
        if cache.get("name") != cfg.name:
            cache.clear()
            torch.cuda.empty_cache()
            cache["name"] = cfg.name
            cache["w"] = tuple(None if w is None else to_dev(w) for w in synth.expert_weights(cfg, threads=16))
        return cache["w"]

    def single_layer(name, cfg, R, path="grouped"):
        wg, wu, wd = weights_of(cfg)
        x = to_dev(synth.hidden0(cfg, 0))
        lg = to_dev(synth.logits(cfg, 0, 0))
        win = 10
        state = torch.empty(moe.moe_stats_state_bytes(1, cfg.E, win), dtype=torch.uint8, device=dev)
        moe.moe_stats_init(state, 1, cfg.E, win)
        bufs = {}
        it = [0]

        def step():
            it[0] += 1
            return moe.moe_layer_forward(x, lg, cfg.k, wg, wu, wd, cfg.act, R, stats_state=state,
                                         stats_dims=(1, cfg.E, win), layer=0, it=it[0], path=path, bufs=bufs,
                                         stream=stream)
        ms = timed(step)
        counts = bufs["counts"].cpu().numpy()
        report(name, cfg, ms, counts, {"replica_budget": R, "gemm_path": path,
                                       "slots_used": int(bufs["disp"]["n_slots"].item())})
        del x, bufs

    def chain(name, cfg, R, graph=False):
        """All L layers of one iteration, statistics and prediction included; the
        time per layer is the chain time over L."""
        cache.clear()
        torch.cuda.empty_cache()
        L, E, k, win = cfg.L, cfg.E, cfg.k, cfg.window
        weights = [tuple(None if w is None else to_dev(w) for w in synth.expert_weights(cfg, l, threads=16))
                   for l in range(L)]
        state = torch.empty(moe.moe_stats_state_bytes(L, E, win), dtype=torch.uint8, device=dev)
        moe.moe_stats_init(state, L, E, win)
        x0 = to_dev(synth.hidden0(cfg, 0))
        # the logits of a chained layer depend on the previous layer's routing: take the
        # routing of an oracle-free first pass on the GPU and keep the logits fixed
        lgs, prev = [], None
        for l in range(L):
            lg = synth.logits(cfg, l, 0, None if prev is None else prev)
            lgs.append(to_dev(lg))
            idx, _ = moe.moe_route(lgs[-1], k)
            prev = idx[:, 0].cpu().numpy()
        bufs = [dict() for _ in range(L)]
        it = [0]

        def step(st=None):
            it[0] += 1
            xx, prev_idx = x0, None
            for l in range(L):
                r = moe.moe_layer_forward(xx, lgs[l], k, *weights[l], cfg.act, R, stats_state=state,
                                          stats_dims=(L, E, win), layer=l, it=it[0], prev_topk_idx=prev_idx,
                                          bufs=bufs[l], stream=stream if st is None else st)
                xx, prev_idx = r["out"], r["idx"]
        ms = timed(step) / L
        counts = np.mean([b["counts"].cpu().numpy() for b in bufs], axis=0)
        extra = {"layers": L, "replica_budget": R, "window": win,
                 "note": "time per layer of the full chain, statistics and prediction included"}
        if graph:
            # the same chain (one iteration index) captured into a HIP graph and
            # replayed: one host call issues every kernel of the chain
            torch.cuda.synchronize()
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            with torch.cuda.stream(side):
                step(side)
            stream.wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(torch.cuda.current_stream())
            extra["graph_ms_per_layer"] = round(timed(g.replay) / L, 4)
            extra["note"] += "; graph_ms_per_layer: the chain replayed from a HIP graph"
            del g
        report(name, cfg, ms, counts, extra)
        del weights, bufs
        torch.cuda.empty_cache()

    C = synth.CONFIGS
    chain("tiny (2-layer chain)", C["tiny"], C["tiny"].R, graph=True)
    single_layer("Mixtral-shaped, R=0", C["mixtral"], 0)
    single_layer("Mixtral-shaped, R=8", C["mixtral"], 8)
    for T in synth.DSV2_T_SWEEP:
        for path in ("grouped", "auto"):
            single_layer(f"DeepSeek-V2-shaped, T={T}", C["dsv2"].with_T(T), 0, path)
    single_layer("DBRX-shaped, R=0", C["dbrx"], 0)
    single_layer("DBRX-shaped, R=16", C["dbrx"], 16)
    chain("PopFetcher-shaped (12-layer chain)", C["popfetcher"], 0)


def stats_bench(moe, synth, torch, np, reps=20):
    """moe_stats of a chained layer (counts, co-occurrence with the previous
    layer, window popularity, conditional matrix, prediction, replicas) on each
    workload's routing shape; median of `reps` event-timed calls."""
    dev = torch.device("cuda:0")
    out = []
    for name, T, E, k, R in (("Mixtral", 8192, 8, 2, 8), ("DBRX", 4096, 16, 4, 16), ("PopFetcher", 16384, 32, 2, 0),
                             ("DeepSeek-V2", 16384, 160, 6, 0), ("DeepSeek-V2", 4096, 160, 6, 0),
                             ("E=256 top-8", 16384, 256, 8, 0)):
        rng = np.random.default_rng(T + E)
        idx = [moe.moe_route(torch.from_numpy((rng.standard_normal((T, E)) -
                                               np.log1p(rng.permutation(E))).astype(np.float32)).to(dev), k)[0]
               for _ in range(2)]
        L, win = 3, 10
        state = torch.empty(moe.moe_stats_state_bytes(L, E, win), dtype=torch.uint8, device=dev)
        moe.moe_stats_init(state, L, E, win)
        o = {n: torch.empty(sz, dtype=dt, device=dev) for n, sz, dt in
             (("c", E, torch.int32), ("p", E, torch.float32), ("P", E * E, torch.float32), ("h", E, torch.float32),
              ("r", E, torch.int32))}
        ts = []
        st = torch.cuda.current_stream()
        for it in range(reps + 3):
            a, b = TimingEvent(), TimingEvent()
            a.record(st)
            moe.moe_stats(state, L, E, win, 1, it, idx[1], idx[0], k, o["c"], o["p"], o["P"], o["h"], R,
                          o["r"] if R else None, st)
            b.record(st)
            torch.cuda.synchronize()
            if it >= 3:
                ts.append(a.elapsed_time(b) * 1e3)
        out.append({"workload": name, "T": T, "E": E, "k": k, "replica_budget": R,
                    "cooccurrence_in": "lds (packed 16-bit)" if E * E <= 32768 else "lds (packed 8-bit)",
                    "us_median": round(float(np.median(ts)), 2)})
    return {"stats": out}


def backward_bench(moe, synth, torch, np, steps=5, warmup=2):
    """The layer's backward pass on the Mixtral-shaped layer (no replication):
    gradients w.r.t. x, the router logits and all expert weights."""
    cfg = synth.CONFIGS["mixtral"]
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    dev = torch.device("cuda:0")

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    wg, wu, wd = (dev_bf16(w) for w in synth.expert_weights(cfg, threads=16))
    x = dev_bf16(synth.hidden0(cfg, 0))
    logits = torch.from_numpy(synth.logits(cfg, 0, 0)).to(dev)
    d_out = torch.randn(T, H, device=dev).to(torch.bfloat16)
    fw = moe.moe_layer_forward(x, logits, k, wg, wu, wd, "swiglu", 0, copy_rows=True)
    ws = torch.empty(moe.moe_backward_workspace_bytes(torch.bfloat16, T, k, H, I, E), dtype=torch.uint8, device=dev)
    out = {}
    stream = torch.cuda.current_stream()

    def run():
        return moe.moe_backward(fw["x_perm"], fw["y_perm"], fw["idx"], fw["w"], fw["inv_pos"], fw["expert_off"],
                                wg, wu, wd, d_out, "swiglu", out, ws, stream)

    for _ in range(warmup):
        out.update(run())
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(steps):
        run()
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    M = T * k
    gemm_flop = 16.0 * M * H * I   # recompute g|u, d_h, d_x_perm, d_Wd, d_Wg|d_Wu
    return {"backward": {"workload": f"Mixtral-shaped layer T={T} H={H} I={I} E={E} k={k} bf16, no replication",
                         "ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
                         "gemm_tflop": round(gemm_flop / 1e12, 3),
                         "gemm_tflops_over_whole_backward": round(gemm_flop / (ms * 1e-3) / 1e12, 1),
                         "workspace_gb": round(ws.numel() / 1e9, 2)}}


def vs_hipblaslt(moe, torch, np, reps=10):
    """The library's GEMMs next to the vendor library on the same dense shapes
    (one expert holding all M = 16384 rows, so no partial tiles): the gate/up GEMM
    (the library's includes the SwiGLU epilogue, torch's is a plain product) and
    the down GEMM.  Times are medians of `reps` launches, HIP events."""
    dev = "cuda"
    M, H, I = 16384, 4096, 14336
    torch.manual_seed(0)
    x = torch.randn(M, H, device=dev).to(torch.bfloat16)
    wg = (torch.randn(1, I, H, device=dev) / H ** 0.5).to(torch.bfloat16)
    wu = (torch.randn(1, I, H, device=dev) / H ** 0.5).to(torch.bfloat16)
    wd = (torch.randn(1, H, I, device=dev) / I ** 0.5).to(torch.bfloat16)
    wgu = torch.cat([wg[0], wu[0]], 0).contiguous()
    h = torch.randn(M, I, device=dev).to(torch.bfloat16)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for s_, e_ in ev:
            s_.record()
            fn()
            e_.record()
        torch.cuda.synchronize()
        return float(np.median([s_.elapsed_time(e_) for s_, e_ in ev]))

    t_gu = timed(lambda: torch.matmul(x, wgu.t()))
    t_d = timed(lambda: torch.matmul(h, wd[0].t()))
    slot_off = torch.tensor([0, M], dtype=torch.int32, device=dev)
    slot_expert = torch.zeros(1, dtype=torch.int32, device=dev)
    n_slots = torch.ones(1, dtype=torch.int32, device=dev)
    ws = torch.empty(moe.moe_expert_ffn_workspace_bytes(torch.bfloat16, M, H, I, 1), dtype=torch.uint8, device=dev)
    y = torch.empty(M, H, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        moe.moe_expert_ffn(x, slot_off, slot_expert, n_slots, wg, wu, wd, "swiglu", "grouped", y, ws)
    torch.cuda.synchronize()
    g1, g2 = [], []
    for _ in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        moe.moe_expert_ffn_profiled(x, slot_off, slot_expert, n_slots, wg, wu, wd, ev, "swiglu", "grouped", y, ws)
        torch.cuda.synchronize()
        g1.append(ev[0].elapsed_time(ev[1]))
        g2.append(ev[1].elapsed_time(ev[2]))
    f_gu, f_d = 2.0 * M * H * 2 * I, 2.0 * M * H * I
    o_gu, o_d = float(np.median(g1)), float(np.median(g2))
    return {"vs_hipblaslt": {
        "shape": "one expert, M=16384, H=4096, I=14336, bf16",
        "gateup": {"hipblaslt_ms": round(t_gu, 4), "hipblaslt_tflops": round(f_gu / t_gu / 1e9, 1),
                   "library_ms": round(o_gu, 4), "library_tflops": round(f_gu / o_gu / 1e9, 1),
                   "note": "the library's launch includes the SwiGLU epilogue; torch's is the plain product"},
        "down": {"hipblaslt_ms": round(t_d, 4), "hipblaslt_tflops": round(f_d / t_d / 1e9, 1),
                 "library_ms": round(o_d, 4), "library_tflops": round(f_d / o_d / 1e9, 1)}}}


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1 "
                                   "(the multi-GPU sharding is a design note, not built)"}))
        sys.exit(2)

    import numpy as np
    import torch

    if a.calibrate_copy:
        x = torch.empty(64 << 20, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        x.fill_(1.0)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "copied 268435456 bytes 3 times"}))
        return

    import mixture_experts_routing_top_amd as moe
    import synth

    if a.crossover:
        crossover(moe, synth, torch, np, tuple(c for c in a.cases.split(",") if c),
                  tuple(p for p in a.paths.split(",") if p))
        return
    if a.vs_hipblaslt:
        print(json.dumps(vs_hipblaslt(moe, torch, np)), flush=True)
        return
    if a.configs:
        configs_bench(moe, synth, torch, np)
        return
    if a.backward:
        print(json.dumps(backward_bench(moe, synth, torch, np)), flush=True)
        return
    if a.stats:
        print(json.dumps(stats_bench(moe, synth, torch, np)), flush=True)
        return
    if a.pipeline:
        print(json.dumps(pipeline_bench(moe, synth, torch, np)), flush=True)
        return
    if a.predict:
        for name, R in (("popfetcher", 8), ("tiny", 4)):
            print(json.dumps(predict_quality(moe, synth, torch, np, name, R)), flush=True)
        return

    cfg = synth.CONFIGS["mixtral"]
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    R = a.replicas
    L, win = 3, 10
    wts = synth.expert_weights(cfg, threads=16)
    x_np = synth.hidden0(cfg, 0)
    prev_logits = synth.logits(cfg, 0, 0)
    logits_np = synth.logits(cfg, 1, 0)  # this workload has no layer-to-layer gamma term
    cpu = None
    if not a.no_cpu_baseline:
        # before anything touches the GPU: the N-core leg forks worker processes
        cpu = cpu_baseline(cfg, x_np, logits_np, wts, prev_logits, R, a.cpu_rows)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def dev_bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    wg, wu, wd = (dev_bf16(w) for w in wts)
    x = dev_bf16(x_np)
    logits = torch.from_numpy(logits_np).to(dev)
    prev_idx, _ = moe.moe_route(torch.from_numpy(prev_logits).to(dev), k)
    stream = torch.cuda.current_stream()
    # cold caches: read a 512 MiB buffer (> the 256 MB MALL plus the L2s) so the
    # step's inputs are evicted and the caches hold clean lines (a write would
    # leave them full of dirty lines that the step then has to write back)
    flush = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    flush_out = torch.empty((), dtype=torch.float32, device=dev)

    def evict(i):
        torch.sum(flush, 0, out=flush_out)

    def make_layer(R_):
        state = torch.empty(moe.moe_stats_state_bytes(L, E, win), dtype=torch.uint8, device=dev)
        moe.moe_stats_init(state, L, E, win)
        bufs = {}

        def step(i, ffn_events=None):
            return moe.moe_layer_forward(x, logits, k, wg, wu, wd, "swiglu", R_, stats_state=state,
                                         stats_dims=(L, E, win), layer=1, it=i, prev_topk_idx=prev_idx,
                                         path=a.path, bufs=bufs, stream=stream, ffn_events=ffn_events)
        return step, state, bufs

    def host_issue_ms(step, first, n=5):
        """Host time to issue one step, median of n; a GPU-side spin keeps the GPU
        busy meanwhile, so no call of the step waits for it."""
        busy = spin_cycles(torch, stream, 5.0)
        ts = []
        for i in range(n):
            torch.cuda.synchronize()
            torch.cuda._sleep(busy)
            t = time.perf_counter()
            step(first + i)
            ts.append(time.perf_counter() - t)
        torch.cuda.synchronize()
        return float(np.median(ts)) * 1e3

    def timed_cold(step, K, first):
        """K steps, each on flushed caches: the 512 MiB flush, then a GPU-side spin
        while the host issues the step (so the events time the GPU, not the host's
        argument marshalling), then the step between two events."""
        ev = [[TimingEvent() for _ in range(5)] for _ in range(K)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            evict(i)
            torch.cuda._sleep(spin)
            ev[i][0].record(stream)
            step(first + i, ffn_events=ev[i][1:4])
            ev[i][4].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = [ev[i][0].elapsed_time(ev[i][4]) for i in range(K)]
        gu = [ev[i][1].elapsed_time(ev[i][2]) for i in range(K)]
        dn = [ev[i][2].elapsed_time(ev[i][3]) for i in range(K)]
        return float(np.mean(ms)), float(np.mean(gu)), float(np.mean(dn)), wall

    def timed_warm(step, K, first):
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record(stream)
        for i in range(K):
            step(first + i)
        end.record(stream)
        torch.cuda.synchronize()
        return start.elapsed_time(end) / K

    def warm_up_cold(step, W):
        """W untimed steps the way the timed ones run (flush, spin, step): the
        first cold steps after warm ones run 1-3% slower than the later ones."""
        for i in range(W):
            evict(i)
            torch.cuda._sleep(spin)
            step(i)
        torch.cuda.synchronize()

    step, state, bufs = make_layer(R)
    step(0)  # loads the kernels and allocates the layer's buffers
    torch.cuda.synchronize()
    # The spin before each cold step only has to outlast the host's issuing of
    # that step: twice its measured issue time, at least 0.3 ms.  A longer idle
    # spin is not neutral: a 1.5 ms spin made the cold step 3-4% slower, all of
    # it in the down GEMM, which starts 3 ms into the step, while back-to-back
    # warm steps do not see it (most likely the power management raising the
    # clock while the chip idles and pulling it back inside the step).
    issue_ms = host_issue_ms(step, 10 ** 5)
    spin_ms = max(0.3, 2.0 * issue_ms)
    spin = spin_cycles(torch, stream, spin_ms)
    warm_up_cold(step, a.warmup)
    # Timed region: exactly K steps (the headline: cold caches before every step).
    ms_step, gateup_ms, down_ms, wall = timed_cold(step, a.steps, a.warmup)
    ms_warm = timed_warm(step, a.steps, a.warmup + a.steps)
    n_slots = int(bufs["disp"]["n_slots"].item())
    # the same layer without replication
    step0, _, bufs0 = make_layer(0)
    warm_up_cold(step0, a.warmup)
    ms_step0, gateup_ms0, _, _ = timed_cold(step0, a.steps, a.warmup)
    ms_warm0 = timed_warm(step0, a.steps, a.warmup + a.steps)
    same_out = bool(torch.equal(bufs0["out"], bufs["out"]))
    del bufs0

    # Per-phase split (diagnostic, outside the timed region): median of 5 passes
    # warm, then 5 cold passes (caches flushed first), each behind a GPU-side spin
    # so the host has issued every phase before the first one starts.
    names = ["route", "stats", "dispatch", "expert_ffn", "combine"]
    samples = {n: [] for n in names}
    cold = {n: [] for n in names}
    spin3 = spin
    for rep in range(10):
        phase_ev = [TimingEvent() for _ in range(6)]
        if rep >= 5:
            evict(rep)
        torch.cuda.synchronize()
        torch.cuda._sleep(spin3)
        phase_ev[0].record(stream)
        idx, w = moe.moe_route(logits, k, bufs["idx"], bufs["w"], stream)
        phase_ev[1].record(stream)
        moe.moe_stats(state, L, E, win, 1, 10 ** 6 + rep, idx, prev_idx, k, bufs["counts"], bufs["p_seq"],
                      bufs["cond"], bufs["pred_next"], R, bufs["replicas"], stream)
        phase_ev[2].record(stream)
        d = moe.moe_dispatch(x, idx, E, bufs["replicas"], E + R, bufs["disp"], bufs["ws_d"], stream, bufs["counts"],
                             copy=False)
        phase_ev[3].record(stream)
        y = moe.moe_expert_ffn(x, d["slot_off"], d["slot_expert"], d["n_slots"], wg, wu, wd, "swiglu",
                               a.path, bufs["y_perm"], bufs["ws_f"], stream, row_src=d["perm_src"])
        phase_ev[4].record(stream)
        moe.moe_combine(y, d["inv_pos"], w, bufs["out"], stream)
        phase_ev[5].record(stream)
        torch.cuda.synchronize()
        for j, n in enumerate(names):
            (samples if rep < 5 else cold)[n].append(phase_ev[j].elapsed_time(phase_ev[j + 1]) * 1e3)
    phase_us = {n: round(float(np.median(v)), 2) for n, v in samples.items()}
    phase_us_cold = {n: round(float(np.median(v)), 2) for n, v in cold.items()}
    del flush

    flops, w_bytes, mem = algorithmic_layer_work(T, H, I, E, k, 3)
    M = T * k
    gateup_flops = 2.0 * M * H * 2 * I
    achieved = gateup_flops / (gateup_ms * 1e-3) / 1e12
    t_roof = flops / (PEAK_BF16_TFLOPS * 1e12) + mem / (PEAK_HBM_GBS * 1e9)
    traffic = measured_traffic(M)
    out = {
        "metric": METRIC,
        "value": round(T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "Mixtral-8x7B-shaped MoE layer", "T": T, "H": H, "I": I, "E": E, "k": k,
                   "act": "swiglu", "replica_budget": R, "slots_used": n_slots, "window": win,
                   "gemm_path": a.path, "stats_chain_layers": L,
                   "timing": "cold: L2 and MALL flushed (512 MiB read) before every timed step",
                   "spin_ms": round(spin_ms, 3), "host_issue_ms": round(issue_ms, 3)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "fused gate/up grouped GEMM (SwiGLU epilogue)",
                     "kernel_ms": round(gateup_ms, 4), "flop_per_launch": gateup_flops},
        "layer_roofline_frac": round(t_roof / (ms_step * 1e-3), 4),
        "layer_roofline_ms": round(t_roof * 1e3, 4),
        "warm": {"ms_per_step": round(ms_warm, 4), "value": round(T / (ms_warm * 1e-3), 1),
                 "note": "K steps back to back, no flush"},
        "replicas_off": {"replica_budget": 0, "ms_per_step": round(ms_step0, 4),
                         "value": round(T / (ms_step0 * 1e-3), 1), "warm_ms_per_step": round(ms_warm0, 4),
                         "gateup_ms": round(gateup_ms0, 4), "out_bit_identical_to_replicated": same_out},
        "down_gemm": {"ms": round(down_ms, 4),
                      "tflops": round(2.0 * M * I * H / (down_ms * 1e-3) / 1e12, 1)},
        "phase_us": phase_us,
        "phase_us_cold": phase_us_cold,
        "memory_phases": memory_phase_summary(T, H, E, k, phase_us, phase_us_cold),
        "wall_s_timed": round(wall, 3),
    }
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out))


if __name__ == "__main__":
    main()
