"""ctypes view of libmoefp8.so (the C ABI declared in include/moefp8.h)."""
from __future__ import annotations

import ctypes
import os

# The in-tree library; MOEFP8_LIB names another build of it (the host-sanitizer build of the CPU
# checks).  There is no fallback: a missing library raises.
LIB_PATH = os.environ.get("MOEFP8_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoefp8.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_UNSUPPORTED_SHAPE = -2
MOE_ERR_WORKSPACE = -3
MOE_ERR_HIP = -4
MOE_ERR_INVALID_DATA = -5

MOE_DTYPE_F32, MOE_DTYPE_BF16, MOE_DTYPE_U8 = 0, 1, 2
MOE_SCALE_F32, MOE_SCALE_UE8M0 = 0, 1
MOE_GROUP_SCORE_TOP2_SUM, MOE_GROUP_SCORE_MAX = 0, 1
MOE_ROUTE_SCORES_GIVEN = 1
MOE_FWD_DETERMINISTIC = 2
MOE_EPI_STORE_F32, MOE_EPI_STORE_BF16, MOE_EPI_SWIGLU_QUANT, MOE_EPI_WEIGHTED_SCATTER_ADD = 0, 1, 2, 3

EXPORTED = ("moe_status_string", "moe_last_error", "fp8_quant_1x128", "fp8_quant_128x128", "moe_route",
            "moe_permute_workspace_size", "moe_permute", "moe_unpermute", "fp8_grouped_gemm_blockscaled",
            "moe_ffn_workspace_size", "moe_ffn_forward", "moe_ffn_forward_stages", "moe_pack_weights",
            "fp8_rmsnorm_quant_1x128", "moe_bias_update", "moe_ffn_forward_noalloc", "moe_padded_rows",
            "fp8_quant_128x1_grouped", "moe_pack_weights_transposed", "fp8_grouped_gemm_wgrad",
            "moe_validation_enabled")
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20
MOE_FWD_STAGE_EVENTS = 6


class MoeCfgC(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int), ("inter", ctypes.c_int), ("n_experts", ctypes.c_int),
                ("top_k", ctypes.c_int), ("n_shared", ctypes.c_int), ("inter_shared", ctypes.c_int),
                ("n_group", ctypes.c_int), ("topk_group", ctypes.c_int), ("group_score", ctypes.c_int),
                ("routed_scale", ctypes.c_float), ("scale_fmt", ctypes.c_int), ("norm_eps", ctypes.c_float)]


class MoeWeightsC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_router", "bias", "w13_q", "w13_s", "w2_q", "w2_s",
                                                "sh_w13_q", "sh_w13_s", "sh_w2_q", "sh_w2_s", "norm_w")]


class MoeEpiC(ctypes.Structure):
    _fields_ = [("h_s", ctypes.c_void_p), ("dst_row", ctypes.c_void_p), ("row_weight", ctypes.c_void_p),
                ("scale_fmt", ctypes.c_int)]


_lib = None


def load() -> ctypes.CDLL:
    """Loads the in-tree library; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(python -m sparse_moe_ffn_sigmoid_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    sig = {
        "moe_status_string": (ctypes.c_char_p, [i]),
        "moe_last_error": (ctypes.c_char_p, []),
        "moe_validation_enabled": (i, []),
        "fp8_quant_1x128": (i, [vp, i, i, i, i, vp, i, vp, i, vp]),
        "fp8_quant_128x128": (i, [vp, i, i, vp, vp, i, vp]),
        "fp8_rmsnorm_quant_1x128": (i, [vp, vp, ctypes.c_float, i, i, i, vp, i, vp, i, vp, i, vp]),
        "moe_bias_update": (i, [vp, i, i, i, ctypes.c_float, vp, vp, vp]),
        "moe_pack_weights": (i, [vp, i, i, i, vp, vp]),
        "moe_route": (i, [vp, vp, vp, i, ctypes.POINTER(MoeCfgC), vp, i, vp, vp, vp]),
        "moe_permute_workspace_size": (sz, [i, i, i]),
        "moe_permute": (i, [vp, i, i, i, vp, vp, vp, vp, i, vp, vp, sz, vp]),
        "moe_unpermute": (i, [vp, i, vp, vp, vp, i, i, i, vp, vp]),
        "fp8_grouped_gemm_blockscaled": (i, [vp, vp, vp, vp, vp, vp, i, i, i, i, i, ctypes.POINTER(MoeEpiC), vp, vp]),
        "moe_ffn_workspace_size": (sz, [i, ctypes.POINTER(MoeCfgC)]),
        "moe_ffn_forward": (i, [vp, i, ctypes.POINTER(MoeCfgC), ctypes.POINTER(MoeWeightsC), vp, sz, vp, vp, vp, vp,
                                i, vp]),
        "moe_ffn_forward_stages": (i, [vp, i, ctypes.POINTER(MoeCfgC), ctypes.POINTER(MoeWeightsC), vp, sz, vp, vp,
                                       vp, vp, i, ctypes.POINTER(ctypes.c_void_p), i, vp]),
        "moe_ffn_forward_noalloc": (i, [vp, i, ctypes.POINTER(MoeCfgC), ctypes.POINTER(MoeWeightsC), vp, vp, vp, vp,
                                        i, vp]),
        "moe_padded_rows": (sz, [i, i]),
        "fp8_quant_128x1_grouped": (i, [vp, i, i, i, i, vp, i, vp, vp, i, vp, i, vp]),
        "moe_pack_weights_transposed": (i, [vp, vp, i, i, i, vp, vp, vp]),
        "fp8_grouped_gemm_wgrad": (i, [vp, vp, vp, vp, vp, i, i, i, i, i, vp, i, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
