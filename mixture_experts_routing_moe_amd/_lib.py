"""ctypes binding of libmoe.so (the C ABI declared in include/moe.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the computation runs in libmoe's kernels.
There is no fallback: if libmoe.so is missing or fails to load, every call
raises.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE = 3
MOE_ERR_HIP = 4
MOE_F32 = 0
MOE_BF16 = 1
MOE_MAX_EXPERTS = 1024
MOE_MAX_TOPK = 64
MOE_DECODE_MAX_T = 64
MOE_MAX_SPLITS = 8
MOE_VERSION = 6
MOE_MAX_GROUPS = 64
MOE_GROUP_LIMITED_GREEDY = 0
MOE_NOAUX_TC = 1

# name -> (restype, argtypes), mirroring include/moe.h
_i32, _i64, _vp, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
_st = ctypes.c_int
SIGNATURES = {
    "moe_version": (ctypes.c_int, []),
    "moe_status_string": (ctypes.c_char_p, [_st]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_route": (_st, [_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp]),
    "moe_route_multihot": (_st, [_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "moe_route_multihot_fused": (_i32, [_i32, _i32]),
    "moe_router_route": (_st, [_st, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "moe_route_grouped": (_st, [_vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                _vp, _vp, _vp, _vp]),
    "moe_align_workspace_size": (_sz, [_i64, _i32, _i32]),
    "moe_route_align": (_st, [_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                              _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_route_align_fused": (_i32, [_i64, _i32, _i32]),
    "moe_ffn_down_combine": (_st, [_i32, _i32, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32,
                                   _i32, _vp, _vp, _vp]),
    "moe_ffn_down_combine_fused": (_i32, [_i32, _i32, _i64, _i32, _i32, _i32, _i32]),
    "moe_tile_schedule_max": (_i64, [_i64, _i32, _i32]),
    "moe_tile_schedule": (_st, [_vp, _i32, _i64, _vp, _vp, _vp, _vp, _vp]),
    "moe_route_align_inverse": (_st, [_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_route_align_noalloc": (_st, [_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp]),
    "moe_route_align_gate_up": (_st, [_vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _i32,
                                      _i32, _vp, _vp, _sz, _vp]),
    "moe_route_align_gate_up_fused": (_i32, [_i64, _i32, _i32, _i32, _i32, _i32, _i32]),
    "moe_align": (_st, [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "moe_align_inverse": (_st, [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                _vp, _vp, _sz, _vp]),
    "moe_indices_to_multihot": (_st, [_vp, _vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp]),
    "moe_multihot_to_indices": (_st, [_vp, _vp, _i64, _i32, _i32, _vp, _vp, _vp]),
    "moe_expert_ffn_workspace_size": (_sz, [_st, _i64, _i32, _i32, _i32, _i32]),
    "moe_expert_ffn": (_st, [_st, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32,
                             _i32, _vp, _vp, _sz, _vp]),
    "moe_expert_ffn_decode": (_st, [_st, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32,
                                    _i32, _i32, _vp, _vp, _sz, _vp]),
    "moe_ffn_gate_up": (_st, [_st, _i32, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _vp,
                              _vp]),
    "moe_ffn_down_splits": (_i32, [_st, _i32, _i64, _i32, _i32, _i32, _i32]),
    "moe_ffn_down": (_st, [_st, _i32, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i32, _i32, _vp,
                           _vp]),
    "moe_combine": (_st, [_st, _vp, _i32, _vp, _vp, _i64, _i32, _i32, _vp, _vp]),
    "moe_route_backward": (_st, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp]),
    "moe_route_grouped_backward": (_st, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp]),
    "moe_router_backward_workspace_size": (_sz, [_i64, _i32, _i32]),
    "moe_router_backward": (_st, [_st, _vp, _vp, _vp, _i64, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "moe_expert_ffn_backward_workspace_size": (_sz, [_i64, _i32, _i32, _i32, _i32]),
    "moe_expert_ffn_backward": (_st, [_st, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64,
                                      _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _sz,
                                      _vp]),
}

_lib = None


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so; raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libmoe.so not built at {LIB_PATH}; run "
                              "`python -m mixture_experts_routing_moe_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def check(status: int, fn: str) -> None:
    if status != MOE_OK:
        l = lib()
        raise MoeError(status, f"{fn}: {l.moe_status_string(status).decode()}: "
                               f"{l.moe_last_error().decode()}")
