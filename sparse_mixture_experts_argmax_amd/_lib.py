"""ctypes view of libmoe.so: the C ABI declared in include/moe.h.

Loading fails loudly if the library has not been built; there is no other
implementation behind these names.
"""
from __future__ import annotations

import ctypes as C
import os

from .source_digest import source_digest

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARGUMENT = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE_TOO_SMALL = 3
MOE_ERR_HIP = 4

MOE_F32 = 0
MOE_BF16 = 1
MOE_ACT_RELU = 0
MOE_ACT_SWIGLU = 1
MOE_POLICY_PRIORITY = 1
MOE_POLICY_REROUTE = 2

SIZE_MAX = (1 << 64) - 1

_p = C.c_void_p
_i64 = C.c_int64
_i32 = C.c_int32
_sz = C.c_size_t


class WsLayout(C.Structure):
    _fields_ = [("slot", _sz), ("expert_count", _sz), ("route_count", _sz),
                ("prob_sum", _sz), ("xbuf", _sz), ("ybuf", _sz), ("row_tok", _sz), ("total", _sz)]


# name -> (restype, argtypes); mirrors include/moe.h
SIGNATURES = {
    "moe_status_string": (C.c_char_p, [C.c_int]),
    "moe_source_digest": (C.c_char_p, []),
    "moe_capacity": (_i64, [_i64, _i32, _i32, C.c_double]),
    "moe_router_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32]),
    "moe_dispatch_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "moe_dispatch_priority_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "moe_router_backward_workspace_bytes": (_sz, [_i64, _i32, _i32]),
    "moe_dispatch_reroute_workspace_bytes": (_sz, [_i64, _i32]),
    "moe_dispatch_reroute": (C.c_int, [_p, C.c_int, _p, _p, _i64, _i32, _i32, _i32, _i32, _i64, _p, _p, _p, _p,
                                       _p, _p, _p, _sz, _p]),
    "moe_combine_backward": (C.c_int, [_p, C.c_int, _p, _p, _p, _p, _i64, _i32, _i32, _i32, _i64, _p, _p, _p]),
    "moe_router_backward": (C.c_int, [_p, C.c_int, _p, _p, _p, _p, _p, _p, _i64, _i32, _i32, _i32,
                                      C.c_float, C.c_float, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_expert_ffn_workspace_bytes": (_sz, [_i32, _i64, _i32, C.c_int]),
    "moe_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32, _i32, _i64, C.c_int, C.c_int]),
    "moe_forward_workspace_layout": (C.c_int, [_i64, _i32, _i32, _i32, _i32, _i64, C.c_int,
                                               C.c_int, C.POINTER(WsLayout)]),
    "moe_router": (C.c_int, [_p, C.c_int, _p, _p, _i64, _i32, _i32, _i32, _p, _p, _p, _p,
                             _p, _p, _p, _sz, _p]),
    "moe_expert_ffn_backward_workspace_bytes": (_sz, [_i32, _i64, _i32, _i32, C.c_int, C.c_int]),
    "moe_expert_ffn_backward": (C.c_int, [_p, C.c_int, _p, _i32, _i64, _i32, _i32, _p, _p, _p, _p, C.c_int,
                                          _p, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_dispatch_backward": (C.c_int, [_p, C.c_int, _p, _p, _i64, _i32, _i32, _i32, _i64, _p, _p, _p]),
    "moe_forward_policy_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32, _i32, C.c_double, C.c_int, C.c_int,
                                                 C.c_int, _i32]),
    "moe_forward_policy": (C.c_int, [_p, C.c_int, _p, _p, _p, _p, _p, _p, _p, C.c_int, _i64, _i32, _i32, _i32, _i32,
                                     C.c_double, C.c_float, C.c_int, _p, _i32, _p, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_router_noalloc": (C.c_int, [_p, C.c_int, _p, _p, _i64, _i32, _i32, _i32, _p, _p, _p, _p,
                                     _p, _p, _p]),
    "moe_router_noalloc_scratch_bytes": (_sz, []),
    "moe_router_noisy": (C.c_int, [_p, C.c_int, _p, _p, _p, _p, _i64, _i32, _i32, _i32, _p, _p, _p,
                                   _p, _p, _p, _sz, _p]),
    "moe_dispatch": (C.c_int, [_p, C.c_int, _p, _i64, _i32, _i32, _i32, _i64, _p, _p, _p, _p,
                               _p, _sz, _p]),
    "moe_dispatch_priority": (C.c_int, [_p, C.c_int, _p, _p, _i64, _i32, _i32, _i32, _i64, _p, _p, _p,
                                        _p, _p, _sz, _p]),
    "moe_expert_ffn": (C.c_int, [_p, C.c_int, _p, _i32, _i64, _i32, _i32, _p, _p, _p, _p, _p,
                                 C.c_int, _p, _p, _sz, _p]),
    "moe_combine": (C.c_int, [_p, C.c_int, _p, _p, _p, _p, _p, _i64, _i32, _i32, _i32, _i64,
                              C.c_float, _p, _p, _p]),
    "moe_forward": (C.c_int, [_p, C.c_int, _p, _p, _p, _p, _p, _p, _p, C.c_int, _i64, _i32, _i32,
                              _i32, _i32, C.c_double, C.c_float, _p, _p, _p, _p, _p, _p, _p, _sz,
                              _p]),
    "moe_forward_noisy": (C.c_int, [_p, C.c_int, _p, _p, _p, _p, _p, _p, _p, _p, _p, C.c_int, _i64, _i32,
                                    _i32, _i32, _i32, C.c_double, C.c_float, _p, _p, _p, _p, _p, _p, _p,
                                    _sz, _p]),
    "moe_forward_staged": (C.c_int, [_p, C.c_int, _p, _p, _p, _p, _p, _p, _p, C.c_int, _i64, _i32,
                                     _i32, _i32, _i32, C.c_double, C.c_float, _p, _p, _p, _p, _p, _p,
                                     _p, _sz, _p, _p]),
}

MOE_STAGE_EVENTS = 6
STAGES = ["router", "dispatch", "expert_gemm1", "expert_gemm2", "combine"]


class MoEError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


def load(path: str = LIB_PATH) -> C.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python sparse_mixture_experts_argmax_amd/build.py` "
            "(the MoE layer has no implementation other than its HIP library)")
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    # a library built from other kernel sources than the tree's would run
    # code that no test in this tree has seen
    built = lib.moe_source_digest().decode()
    here = source_digest()
    if built != here:
        raise RuntimeError(
            f"{path} was built from other sources (digest {built}, the tree's csrc/ is {here}): rebuild it "
            "with `python sparse_mixture_experts_argmax_amd/build.py`")
    return lib


LIB = load()


def status_string(status: int) -> str:
    return LIB.moe_status_string(status).decode()


def check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoEError(fn, status, status_string(status))
