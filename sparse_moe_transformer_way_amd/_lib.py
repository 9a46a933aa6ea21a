"""ctypes loading of libmoe_mi355x.so and the C declarations of include/moe.h.

The library must have been built (python sparse_moe_transformer_way_amd/build.py);
there is no fallback of any kind: a missing library raises at import.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe_mi355x.so")

MOE_OK = 0
MOE_ERR_INVALID_ARGUMENT = 1
MOE_ERR_UNSUPPORTED = 2
MOE_ERR_WORKSPACE_TOO_SMALL = 3
MOE_ERR_HIP = 4

MOE_F32 = 0
MOE_BF16 = 1
MOE_FP8_E4M3 = 2

MOE_NOALLOC_SCRATCH_BYTES = 16 << 20  # scratch of moe_layer_forward_noalloc per GPU


class LayerDesc(ctypes.Structure):
    """moe_layer_desc_t."""
    _fields_ = [
        ("d_model", ctypes.c_int32),
        ("d_ffn", ctypes.c_int32),
        ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32),
        ("act_dtype", ctypes.c_int32),
        ("weight_dtype", ctypes.c_int32),
    ]


_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_desc = ctypes.POINTER(LayerDesc)

# name -> (restype, argtypes), in the order of include/moe.h
SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_i32]),
    "moe_version": (_i32, []),
    "moe_default_tile_m": (_i32, [_desc, _i32]),
    "moe_max_permuted_rows": (ctypes.c_int64, [_desc, _i32, _i32]),
    "moe_workspace_size": (ctypes.c_size_t, [_desc, _i32, _i32]),
    "moe_router_topk": (_i32, [_desc, _i32, _p, _p, _p, _p, _p, _p]),
    "moe_permute": (_i32, [_desc, _i32, _i32, _p, _p, _p, _p, _p, _p]),
    "moe_expert_gate_up": (_i32, [_desc, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p]),
    "moe_expert_down": (_i32, [_desc, _i32, _i32, _p, _p, _p, _p, _p, _p]),
    "moe_grouped_swiglu": (_i32, [_desc, _i32, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "moe_combine": (_i32, [_desc, _i32, _p, _p, _p, _p, _p, _p]),
    "moe_rmsnorm": (_i32, [_i32, _i32, _i32, _p, ctypes.c_float, _p, _p]),
    "moe_layer_forward": (_i32, [_desc, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                 ctypes.c_size_t, _p]),
    "moe_layer_forward_timed": (_i32, [_desc, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                       ctypes.c_size_t, _p, _p]),
    "moe_layer_forward_noalloc": (_i32, [_desc, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "moe_block_workspace_size": (ctypes.c_size_t, [_desc, _i32]),
    "moe_block_forward": (_i32, [_desc, _i32, _p, ctypes.c_float, _p, _p, _p, _p, _p, _p, _p, _p,
                                 ctypes.c_size_t, _p]),
    "moe_quantize_fp8": (_i32, [ctypes.c_int64, _i32, _p, _p, _p, _p]),
    "moe_expert_gate_up_fp8": (_i32, [_desc, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "moe_expert_down_fp8": (_i32, [_desc, _i32, _p, _p, _p, _p, _p, _p, _p]),
    "moe_layer_forward_fp8": (_i32, [_desc, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                     _p, ctypes.c_size_t, _p]),
    "moe_backward_workspace_size": (ctypes.c_size_t, [_desc, _i32]),
    "moe_layer_backward": (_i32, [_desc, _i32, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                  ctypes.c_size_t, _p]),
}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build it with `python sparse_moe_transformer_way_amd/build.py` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = load()


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        name = lib.moe_status_string(status).decode()
        super().__init__(f"{fn} returned {name} ({status})")
        self.status = status
