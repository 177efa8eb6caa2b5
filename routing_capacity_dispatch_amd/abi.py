"""ctypes mirror of include/moe.h and loader of the in-tree libmoe.so.

Argument marshalling only: every step of the branch runs in the HIP library.
Loading fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB selects another build of the library (e.g. the host-sanitized one)
LIB_PATH = os.environ.get("MOE_LIB") or os.path.join(_PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED",
                3: "MOE_ERR_WORKSPACE", 4: "MOE_ERR_HIP"}


class MoeConfig(C.Structure):
    _fields_ = [
        ("T", C.c_int64),
        ("d_model", C.c_int32), ("d_latent", C.c_int32), ("n_experts", C.c_int32),
        ("n_pools", C.c_int32), ("top_k", C.c_int32), ("d_ff", C.c_int32),
        ("n_shared", C.c_int32), ("d_ff_shared", C.c_int32), ("n_waves", C.c_int32),
        ("send_cap_num", C.c_int32), ("send_cap_den", C.c_int32),
        ("recv_cap_num", C.c_int32), ("recv_cap_den", C.c_int32),
        ("cap_send_rows", C.c_int64), ("cap_recv_rows", C.c_int64),
        ("dtype", C.c_int32), ("reserved", C.c_int32),
    ]


class MoePlan(C.Structure):
    _fields_ = [(n, C.c_int64) for n in (
        "tokens_per_wave", "cap_send", "cap_recv", "experts_per_pool", "elem_bytes",
        "row_bytes", "pool_block_bytes", "ids_offset", "pools_bytes", "expert_out_bytes",
        "max_expert_rows", "dispatch_ws_bytes", "experts_ws_bytes", "forward_ws_bytes",
        "dropless_rows", "dropless_dispatch_ws_bytes", "dropless_experts_ws_bytes",
        "dropless_forward_ws_bytes", "backward_rows", "experts_bwd_ws_bytes",
        "backward_ws_bytes", "dropless_backward_rows", "dropless_experts_bwd_ws_bytes",
        "dropless_backward_ws_bytes")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class MoeWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "w_latent", "w_router", "router_bias", "w_gate", "w_up", "w_down", "w_up_proj",
        "ws_gate", "ws_up", "ws_down")]


class MoeTaps(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "logits", "topk_idx", "gates", "pool_slot", "recv_slot", "pool_count",
        "expert_count", "bank_rows", "z", "pools", "expert_out", "y_latent")]


class MoeDroplessTaps(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "logits", "topk_idx", "gates", "row_of", "expert_offsets", "z", "xs", "expert_out",
        "y_latent")]


# exported symbols and their signatures
_P = C.c_void_p
SIGNATURES = {
    "moe_status_string": (C.c_char_p, [C.c_int]),
    "moe_version": (C.c_int32, []),
    "moe_make_plan": (C.c_int, [C.POINTER(MoeConfig), C.POINTER(MoePlan)]),
    "moe_route": (C.c_int, [C.POINTER(MoeConfig), _P, _P, _P, _P, _P]),
    "moe_router_bias_ws_bytes": (C.c_int, [C.POINTER(MoeConfig), C.c_int32, C.POINTER(C.c_size_t)]),
    "moe_router_bias_update": (C.c_int, [C.POINTER(MoeConfig), _P, C.c_int32, _P, _P, _P, _P,
                                         C.c_size_t, _P]),
    "moe_router_bias_stage_count": (C.c_int32, []),
    "moe_router_bias_update_profiled": (C.c_int, [C.POINTER(MoeConfig), _P, C.c_int32, _P, _P, _P, _P,
                                                  C.c_size_t, _P, _P, C.c_int32]),
    "moe_dispatch": (C.c_int, [C.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                               _P, C.c_size_t, _P]),
    "moe_dispatch_noalloc": (C.c_int, [C.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_dispatch_noalloc_scratch_bytes": (C.c_int64, []),
    "moe_experts": (C.c_int, [C.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P, _P,
                              C.c_size_t, _P]),
    "moe_combine": (C.c_int, [C.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P]),
    "moe_forward": (C.c_int, [C.POINTER(MoeConfig), C.POINTER(MoeWeights), _P, _P,
                              C.POINTER(MoeTaps), _P, _P, C.c_size_t, _P]),
    "moe_forward_stage_count": (C.c_int32, []),
    "moe_forward_profiled": (C.c_int, [C.POINTER(MoeConfig), C.POINTER(MoeWeights), _P, _P,
                                       C.POINTER(MoeTaps), _P, _P, C.c_size_t, _P,
                                       C.POINTER(C.c_void_p), C.c_int32]),
    "moe_dispatch_dropless": (C.c_int, [C.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P,
                                        C.c_size_t, _P]),
    "moe_experts_dropless": (C.c_int, [C.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P,
                                       C.c_size_t, _P]),
    "moe_combine_dropless": (C.c_int, [C.POINTER(MoeConfig), _P, _P, _P, _P, _P]),
    "moe_forward_dropless": (C.c_int, [C.POINTER(MoeConfig), C.POINTER(MoeWeights), _P, _P,
                                       C.POINTER(MoeDroplessTaps), _P, _P, C.c_size_t, _P]),
    "moe_forward_dropless_stage_count": (C.c_int32, []),
    "moe_forward_dropless_profiled": (C.c_int, [C.POINTER(MoeConfig), C.POINTER(MoeWeights),
                                                _P, _P, C.POINTER(MoeDroplessTaps), _P, _P,
                                                C.c_size_t, _P, C.POINTER(C.c_void_p),
                                                C.c_int32]),
    "moe_combine_backward": (C.c_int, [C.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "moe_experts_backward": (C.c_int, [C.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P, _P, _P,
                                       _P, _P, _P, C.c_size_t, _P]),
    "moe_dispatch_backward": (C.c_int, [C.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P]),
    "moe_route_backward": (C.c_int, [C.POINTER(MoeConfig), _P, _P, _P, _P, _P]),
    "moe_backward_routed": (C.c_int, [C.POINTER(MoeConfig), C.POINTER(MoeWeights),
                                      C.POINTER(MoeTaps), _P, _P, _P, _P, _P, _P, _P,
                                      C.c_size_t, _P]),
    "moe_backward_routed_stage_count": (C.c_int32, []),
    "moe_combine_backward_dropless": (C.c_int, [C.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P]),
    "moe_experts_backward_dropless": (C.c_int, [C.POINTER(MoeConfig), _P, _P, _P, _P, _P, _P, _P,
                                                _P, _P, _P, _P, C.c_size_t, _P]),
    "moe_dispatch_backward_dropless": (C.c_int, [C.POINTER(MoeConfig), _P, _P, _P, _P]),
    "moe_backward_dropless": (C.c_int, [C.POINTER(MoeConfig), C.POINTER(MoeWeights),
                                        C.POINTER(MoeDroplessTaps), _P, _P, _P, _P, _P, _P, _P,
                                        C.c_size_t, _P]),
    "moe_backward_dropless_profiled": (C.c_int, [C.POINTER(MoeConfig), C.POINTER(MoeWeights),
                                                 C.POINTER(MoeDroplessTaps), _P, _P, _P, _P, _P,
                                                 _P, _P, C.c_size_t, _P, C.POINTER(C.c_void_p),
                                                 C.c_int32]),
    "moe_backward_routed_profiled": (C.c_int, [C.POINTER(MoeConfig), C.POINTER(MoeWeights),
                                               C.POINTER(MoeTaps), _P, _P, _P, _P, _P, _P, _P,
                                               C.c_size_t, _P, C.POINTER(C.c_void_p),
                                               C.c_int32]),
}

STAGES = ["latent", "router", "topk", "assign", "scatter", "recv_bin", "expert_rows",
          "expert_gate_up", "expert_down", "combine", "shared_gate_up", "output"]
DROPLESS_STAGES = ["latent", "router", "topk", "sort", "scatter", "tiles", "expert_gate_up",
                   "expert_down", "combine", "shared_gate_up", "output"]
BIAS_STAGES = ["bias_range", "bias_hist", "bias_quantile", "bias_mean"]
BACKWARD_STAGES = ["combine_bwd", "layout", "gather", "dh", "swiglu_bwd", "du", "dw_down",
                   "dw_gate", "dw_up", "dispatch_bwd", "route_bwd"]

_lib = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load libmoe.so (cached).  Raises if it is missing: there is no fallback."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing; build it with `python -m routing_capacity_dispatch_amd.build`")
    lib = C.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)}")


def check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status)
