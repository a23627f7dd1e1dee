"""Loads libmoe_mi355x.so and declares the C signatures of include/moe.h."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")
_lib = None

_p, _i, _i64, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "moe_route": (_i, [_p, _i64, _i, _i, _p, _p, _p, _p]),
    "moe_stats_state_bytes": (_sz, [_i, _i, _i]),
    "moe_stats_init": (_i, [_p, _sz, _i, _i, _i, _p]),
    "moe_stats": (_i, [_p, _sz, _i, _i, _i, _i, _i64, _p, _p, _i64, _i, _p, _p, _p, _p, _i, _p, _p, _p]),
    "moe_stats_load_state": (_i, [_p, _sz, _i, _i, _i, _i, _i64, ctypes.c_double, _p, _p, _p, _p]),
    "moe_plan_replicas": (_i, [_p, _i, _i64, _i, _p, _p, _p]),
    "moe_prediction_quality": (_i, [_p, _p, _i, _p, _i, _p, _p]),
    "moe_dispatch_workspace_bytes": (_sz, [_i64, _i, _i]),
    "moe_dispatch": (_i, [_p, _i, _i64, _i, _p, _i, _i, _p, _p, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p, _p]),
    "moe_dispatch_noalloc": (_i, [_p, _i, _i64, _i, _p, _i, _i, _p, _p, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "moe_expert_ffn_workspace_bytes": (_sz, [_i, _i64, _i, _i, _i]),
    "moe_expert_ffn": (_i, [_p, _p, _i64, _i, _i64, _i, _i, _i, _p, _p, _p, _i, _p, _p, _p, _i, _i, _p, _p, _sz, _p,
                            _p]),
    "moe_expert_ffn_profiled": (_i, [_p, _p, _i64, _i, _i64, _i, _i, _i, _p, _p, _p, _i, _p, _p, _p, _i, _i, _p, _p,
                                     _sz, _p,
                                     _p, _p]),
    "moe_combine": (_i, [_p, _i, _i64, _p, _p, _i64, _i, _i, _p, _p, _p]),
    "moe_backward_workspace_bytes": (_sz, [_i, _i64, _i, _i, _i, _i, _i]),
    "moe_backward": (_i, [_p, _p, _i, _i64, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _i, _p, _p, _p, _p, _p, _p,
                          _p, _sz, _p]),
    "moe_check_device_error": (_i, [_p, _p, _p]),
    "moe_status_string": (ctypes.c_char_p, [_i]),
    "moe_last_error": (ctypes.c_char_p, []),
}


class MoEError(RuntimeError):
    def __init__(self, call, status, message):
        self.call, self.status = call, status
        super().__init__(f"{call} failed with status {status}: {message}")


def lib():
    """The loaded library.  Raises if it has not been built: there is no fallback path."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m mixture_experts_routing_top_amd.build` "
                               "(the MoE layer has no non-HIP fallback)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib
