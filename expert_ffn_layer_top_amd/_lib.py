"""ctypes binding of libmoe_mi355x.so (the C ABI in include/moe_mi355x.h).

Loads the in-tree library built by `python -m expert_ffn_layer_top_amd.build`.  There is no
fallback: if the library is missing or lacks a symbol, importing this module raises.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

_i = ctypes.c_int
_sz = ctypes.c_size_t
_p = ctypes.c_void_p

# name -> (restype, argtypes); the order and meaning of arguments follow include/moe_mi355x.h
SIGNATURES = {
    "moe_abi_version": (_i, []),
    "moe_status_string": (ctypes.c_char_p, [_i]),
    "moe_last_error_string": (ctypes.c_char_p, []),
    "moe_router_project": (_i, [_p, _p, _i, _i, _i, _p, _p]),
    "moe_router_bwd_workspace_bytes": (_sz, [_i, _i, _i]),
    "moe_router_project_bwd": (_i, [_p, _p, _p, _i, _i, _i, _p, _p, _p, _sz, _p]),
    "moe_route_workspace_bytes": (_sz, [_i, _i, _i]),
    "moe_route_topk": (_i, [_p, _i, _i, _i, _p, _p, _p, _p, _p, _p, _i, _p, _p, _p, _sz, _p]),
    "moe_route_topk_noalloc": (_i, [_p, _i, _i, _i, _p, _p, _p, _p, _p, _p, _i, _p, _p, _p]),
    "moe_route_topk_bwd": (_i, [_p, _p, _p, _i, _i, _i, _p, _p]),
    "moe_route_balance_workspace_bytes": (_sz, [_i, _i]),
    "moe_route_balance": (_i, [_p, _p, _i, _i, _i, _p, _p, _p, _sz, _p]),
    "moe_route_topk_bwd_balance": (_i, [_p, _p, _p, _p, _p, ctypes.c_float, _i, _i, _i, _p, _p]),
    "moe_permute": (_i, [_i, _p, _p, _p, _i, _i, _i, _p, _p, _p]),
    "moe_unpermute_combine": (_i, [_p, _p, _p, _i, _i, _i, _p, _p]),
    "moe_unpermute_combine_bwd": (_i, [_p, _p, _p, _p, _i, _i, _i, _p, _p, _p]),
    "moe_unpermute_combine_bwd_mx": (_i, [_p, _p, _p, _p, _i, _i, _i, _p, _p, _p, _p, _p]),
    "moe_permute_bwd": (_i, [_p, _p, _i, _i, _i, _p, _p, _p]),
    "moe_permute_bwd_router": (_i, [_p, _p, _i, _i, _i, _p, _p, _i, _p, _p, _sz, _p]),
    "mxfp8_quantize": (_i, [_p, _i, _i, _i, _i, _i, _p, _p, _p]),
    "mxfp8_quantize_both": (_i, [_p, _i, _i, _i, _p, _p, _p, _p, _p]),
    "mxfp8_quantize_grouped": (_i, [_p, _p, _p, _p, _i, _i, _i, _p, _p, _p]),
    "mxfp8_quantize_grouped_gated": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _p, _p, _p]),
    "mxfp8_quantize_rows_grouped": (_i, [_p, _p, _p, _i, _i, _i, _p, _p, _p, _p, _p]),
    "moe_permute_quant_mx": (_i, [_p, _p, _i, _i, _i, _p, _p, _p]),
    "mxfp8_quantize_gemm": (_i, [_p, _i, _i, _i, _p, _p, _p]),
    "mxfp8_scales_to_gemm": (_i, [_p, _i, _i, _i, _p, _p]),
    "moe_mx_pad_cap": (_i, [_i, _i]),
    "moe_gg_workspace_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "moe_grouped_gemm_swiglu": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                     _p, _p, _p, _p, _p, _sz, _p]),
    "moe_grouped_gemm_gate_up": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "moe_grouped_gemm_down": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _sz, _p]),
    "moe_grouped_gemm_down_mx": (_i, [_i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p]),
    "moe_grouped_gemm_swiglu_bwd": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p,
                                         _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                         _sz, _p]),
    "moe_grouped_gemm_dgrad_down": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p, _p]),
    "moe_grouped_gemm_wgrad_down": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p]),
    "moe_grouped_gemm_dgrad_gate_up": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                            _p, _p]),
    "moe_grouped_gemm_wgrad_gate_up": (_i, [_i, _i, _i, _i, _i, _p, _p, _p, _p, _p, _p, _p, _p, _p,
                                            _p, _p]),
}


class MoeError(RuntimeError):
    def __init__(self, fn, status, text):
        super().__init__(f"{fn} failed: status {status} ({text})")
        self.status = status


def _init_torch_device():
    """Creates torch's HIP context before the library registers its kernels.

    The library shares torch's HIP runtime (torch/lib/libamdhip64.so).  With that runtime, kernels
    registered before torch's lazy device initialisation were not found at launch ("no ROCm-capable
    device is detected"), while the same library loaded after it ran correctly, so the context is
    created first.  Without a GPU this does nothing (host-only checks still load the library).
    """
    import torch
    if torch.cuda.is_available():
        torch.cuda.init()
        torch.empty(1, device="cuda")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m expert_ffn_layer_top_amd.build`")
    _init_torch_device()
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)            # AttributeError if the symbol is missing
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def call(name, *args):
    """Calls `name` and raises MoeError on a nonzero status."""
    st = getattr(lib, name)(*args)
    if st != 0:
        raise MoeError(name, st, lib.moe_last_error_string().decode())
    return st
