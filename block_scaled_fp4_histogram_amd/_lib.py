"""ctypes binding of libmoe_gfx950.so (the C ABI in include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes as C
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB_PATH points at another build of the same library (e.g. a variant being measured)
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(_PKG, "libmoe_gfx950.so")

# Every function include/moe.h declares, with (restype, argtypes).
_vp, _i, _f, _sz = C.c_void_p, C.c_int, C.c_float, C.c_size_t
SIGNATURES = {
    "moe_plan": (_i, [_i, _i, _i, _i, _f, _i, _i, _i, C.POINTER(_vp)]),
    "moe_plan_destroy": (None, [_vp]),
    "moe_scratch_bytes": (_sz, [_vp, _i, _i]),
    "moe_prepare_weights": (_i, [_vp, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, C.POINTER(_vp)]),
    "moe_unpack_weights": (_i, [_vp, _vp]),
    "moe_experts_destroy": (None, [_vp]),
    "moe_run": (_i, [_vp, _vp, _i, _vp, _vp, _vp, _vp, _i, _i, _vp, _sz, _vp]),
    "moe_run_noalloc": (_i, [_vp, _vp, _i, _vp, _vp, _vp, _vp, _i, _i, _vp]),
    "moe_last_error": (C.c_char_p, []),
    "moe_plan_capacity": (_i, [_vp, _i, C.POINTER(_i)]),
    "moe_plan_set_sequence": (_i, [_vp, _i, _i]),
    "moe_plan_sequence": (_i, [_vp, _i]),
    "moe_plan_autotune": (_i, [_vp, _vp, _i, C.POINTER(_i), _i, _i, _i, _vp, C.POINTER(_f)]),
    "moe_plan_autotune_batch": (_i, [_vp, _vp, _i, _vp, _vp, _vp, _i, _i, _i, _vp, C.POINTER(_f)]),
    "moe_plan_set_combine": (_i, [_vp, _i, _i]),
    "moe_plan_combine": (_i, [_vp, _i]),
    "moe_plan_save_tuning": (_i, [_vp, C.c_char_p]),
    "moe_plan_load_tuning": (_i, [_vp, C.c_char_p]),
    "moe_plan_set_router_weight_on_input": (_i, [_vp, _i]),
    "moe_plan_set_swiglu_oai": (_i, [_vp, C.c_float, C.c_float]),
    "moe_plan_set_activation": (_i, [_vp, _i]),
    "moe_plan_enable_stage_timing": (_i, [_vp, _i]),
    "moe_plan_stage_times": (_i, [_vp, C.POINTER(_f), _i, C.POINTER(_i)]),
    "moe_ep_remap": (_i, [_vp, _vp, _i, _i, C.c_longlong, _i, _vp, _vp, _vp]),
    "moe_debug_route": (_i, [_vp, _vp, _i, _vp, _i, _vp, _sz, _vp, _vp, _vp, _vp, _vp]),
    "moe_debug_quant_mxfp8_bf16": (_i, [_vp, _i, _i, _vp, _vp, _vp]),
    "moe_debug_quant_mxfp8_f32": (_i, [_vp, _i, _i, _vp, _vp, _vp]),
}


class MoeTier(C.Structure):
    _fields_ = [("experts", C.c_void_p), ("expert_map", C.c_void_p)]


_lib = None


def load():
    """Load the library once. Raises ImportError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with block_scaled_fp4_histogram_amd/build.py "
                              "(or __graft_entry__.build())")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib
