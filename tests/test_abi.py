"""The C-ABI library on the CPU: it loads, exports every entry point the header
declares, and rejects bad arguments before anything reaches the GPU.  No
compute call is made here."""
import ctypes
import os
import re

import pytest

import mixture_experts_routing_top_amd as moe
from mixture_experts_routing_top_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _lib():
    if not os.path.exists(_native.LIB_PATH):
        from mixture_experts_routing_top_amd import build
        build.build()
    return _native.lib()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = _declared()
    for n in ("moe_route", "moe_stats", "moe_dispatch", "moe_expert_ffn", "moe_combine"):
        assert n in names


def test_every_declared_symbol_is_exported_and_bound():
    lib = _lib()
    for name in _declared():
        assert hasattr(lib, name), name
        assert name in _native.SIGNATURES, name


def test_library_is_gfx950_code_object():
    data = open(_native.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_status_strings():
    lib = _lib()
    assert lib.moe_status_string(0) == b"ok"
    assert lib.moe_status_string(-3) == b"workspace or state too small"
    assert lib.moe_status_string(-5) == b"the device check flagged invalid input"


N = None


@pytest.mark.parametrize("call,args,status,msg", [
    ("moe_route", (N, 10, 0, 2, N, N, N, N), -1, "E=0"),
    ("moe_route", (N, 10, 300, 2, N, N, N, N), -2, "E=300"),
    ("moe_route", (N, 10, 8, 9, N, N, N, N), -1, "k=9"),
    ("moe_route", (N, 10, 8, 2, N, N, N, N), -1, "null"),
    ("moe_route", (N, -1, 8, 2, N, N, N, N), -1, "T="),
    ("moe_stats", (1, 1 << 20, 2, 8, 10, 2, 0, 1, N, 0, 2, N, N, N, N, 0, N, N, N), -1, "layer=2"),
    ("moe_stats", (1, 8, 2, 8, 10, 1, 0, 1, N, 0, 2, N, N, N, N, 0, N, N, N), -3, "too small"),
    ("moe_stats", (1, 1 << 20, 2, 8, 10, 1, 0, 1, N, 100, 2, N, N, N, N, 0, N, N, N), -1, "prev_topk_idx"),
    ("moe_stats_init", (N, 0, 2, 8, 10, N), -1, "null state"),
    ("moe_dispatch", (16, 0, 10, 64, 16, 2, 8, N, N, 0, 8, 16, 16, 16, 16, 16, 16, 16, 16, 0, N, N), -3, "workspace"),
    ("moe_dispatch", (1, 1, 10, 7, 1, 2, 8, N, N, 0, 8, 1, 1, 1, 1, 1, 1, 1, 1, 1 << 20, N, N), -1, "multiple of 16"),
    ("moe_dispatch", (1, 0, 10, 64, 1, 2, 8, N, N, 0, 4, 1, 1, 1, 1, 1, 1, 1, 1, 1 << 20, N, N), -1, "max_slots"),
    ("moe_dispatch", (8, 0, 10, 64, 8, 2, 8, N, N, 0, 8, 8, 8, 8, 8, 8, 8, 8, 8, 1 << 20, N, N), -1, "aligned"),
    ("moe_dispatch", (16, 0, 10, 64, 16, 2, 8, N, N, 5, 12, 16, 16, 16, 16, 16, 16, 16, 16, 1 << 20, N, N), -1,
     "replica_budget"),
    ("moe_dispatch", (16, 0, 10, 64, 16, 2, 8, N, 16, 2, 12, 16, 16, 16, 16, 16, 16, 16, 16, 1 << 20, N, N), -1,
     "replica_budget"),
    ("moe_expert_ffn", (16, N, 0, 1, 100, 96, 128, 8, 16, 16, 16, 8, 16, 16, 16, 0, 1, 16, 16, 1 << 30, N, N), -2, "multiples of 64"),
    ("moe_expert_ffn", (16, N, 0, 1, 100, 128, 128, 8, 16, 16, 16, 8, 16, N, 16, 0, 1, 16, 16, 1 << 30, N, N), -1, "w_up"),
    ("moe_expert_ffn", (16, N, 0, 1, 100, 128, 128, 8, 16, 16, 16, 8, 16, 16, 16, 1, 1, 16, 16, 1 << 30, N, N), -1, "GELU"),
    ("moe_expert_ffn", (16, N, 0, 1, 100, 128, 128, 8, 16, 16, 16, 8, 16, 16, 16, 0, 1, 16, 16, 10, N, N), -3, "workspace"),
    # a gathered input (row_src given) of 2^40 rows: offsets beyond 31 bits
    ("moe_expert_ffn", (16, 16, 1 << 40, 1, 100, 128, 128, 8, 16, 16, 16, 8, 16, 16, 16, 0, 1, 16, 16, 1 << 30, N, N),
     -2, "gathered input"),
    # 2^27 rows x 2^21 columns: more blocks than 32-bit grid indexing covers
    ("moe_expert_ffn", (16, N, 0, 1, 1 << 27, 64, 1 << 21, 8, 16, 16, 16, 8, 16, 16, 16, 0, 1, 16, 16, 1 << 62, N, N), -2,
     "32-bit grid"),
    ("moe_stats_load_state", (1, 1 << 20, 2, 8, 10, 0, 0, 1.5, N, N, N, N), -1, "decay"),
    ("moe_stats_load_state", (1, 1 << 20, 2, 8, 10, 2, 0, 0.9, N, N, N, N), -1, "layer=2"),
    ("moe_stats_load_state", (1, 8, 2, 8, 10, 0, 0, 0.9, N, N, N, N), -3, "too small"),
    ("moe_stats_load_state", (1, 1 << 20, 2, 8, 10, 0, -1, 0.9, N, N, N, N), -1, "iter"),
    ("moe_plan_replicas", (16, 0, 10, 2, N, 16, N), -1, "E=0"),
    ("moe_plan_replicas", (16, 300, 10, 2, N, 16, N), -2, "E=300"),
    ("moe_plan_replicas", (16, 8, -1, 2, N, 16, N), -1, "total"),
    ("moe_plan_replicas", (16, 8, 10, 5000, N, 16, N), -1, "replica_budget"),
    ("moe_plan_replicas", (16, 8, 10, 2, N, N, N), -1, "null"),
    ("moe_prediction_quality", (16, 16, 8, N, 0, 16, N), -1, "top_n"),
    ("moe_prediction_quality", (16, N, 8, N, 5, 16, N), -1, "null"),
    ("moe_prediction_quality", (16, 16, 257, N, 5, 16, N), -2, "E=257"),
    ("moe_backward", (16, 16, 1, 10, 2, 96, 128, 8, 16, 16, 16, 16, 16, 16, 16, 0, 16, 16, 16, 16, 16, 16, 16,
                      1 << 40, N), -2, "multiples of 64"),
    ("moe_backward", (16, 16, 1, 10, 2, 128, 128, 8, 16, 16, 16, 16, 16, N, 16, 0, 16, 16, 16, 16, 16, 16, 16,
                      1 << 40, N), -1, "w_up"),
    ("moe_backward", (16, 16, 1, 10, 2, 128, 128, 8, 16, 16, 16, 16, 16, 16, 16, 0, 16, 16, 16, 16, 16, 16, 16,
                      10, N), -3, "workspace"),
    ("moe_backward", (16, 16, 1, 10, 9, 128, 128, 8, 16, 16, 16, 16, 16, 16, 16, 0, 16, 16, 16, 16, 16, 16, 16,
                      1 << 40, N), -1, "k=9"),
    # 16 experts with I = 2^20: the weight-gradient grid exceeds 32-bit indexing
    ("moe_backward", (16, 16, 1, 10, 2, 64, 1 << 20, 16, 16, 16, 16, 16, 16, 16, 16, 0, 16, 16, 16, 16, 16, 16, 16,
                      1 << 62, N), -2, "32-bit grid"),
    ("moe_combine", (16, 1, 10, 16, 16, 10, 9, 64, 16, N, N), -1, "k=9"),
    ("moe_combine", (16, 1, 10, 16, 16, 10, 2, 12, 16, N, N), -1, "multiple of 16"),
    ("moe_check_device_error", (N, N, N), -1, "null check"),
    ("moe_expert_ffn_profiled", (16, N, 0, 1, 100, 128, 128, 8, 16, 16, 16, 8, 16, 16, 16, 0, 1, 16, 16, 1 << 30, N, N, N),
     -1, "three events"),
])
def test_argument_errors_are_reported_before_any_hip_call(call, args, status, msg):
    lib = _lib()
    cargs = [None if a is None else a for a in args]
    rc = getattr(lib, call)(*cargs)
    assert rc == status, (rc, lib.moe_last_error())
    assert msg in lib.moe_last_error().decode()


def test_workspace_queries():
    lib = _lib()
    assert lib.moe_stats_state_bytes(12, 32, 10) >= 4 * (10 * 12 * 32 + 10 * 11 * 32 * 32)
    assert lib.moe_stats_state_bytes(0, 32, 10) == 0
    assert lib.moe_dispatch_workspace_bytes(8192, 2, 8) >= 4 * 32 * 8
    assert lib.moe_expert_ffn_workspace_bytes(1, 16384, 4096, 14336, 16) >= 16384 * 14336 * 2


def test_binding_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        moe.moe_route(torch.zeros((4, 8)), 2)


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "mixture_experts_routing_top_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "moe_oracle" not in text and "liboracle" not in text, f
