"""ctypes declarations of the C ABI in include/moe.h (libmoe.so, built in-tree).

Loading fails loudly when the library has not been built: there is no other
implementation to fall back on.
"""
import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_LIB_PATH names another build of the same library (the host-sanitised
# build of the CPU sanitizer test); by default the in-tree libmoe.so
LIB_PATH = os.environ.get("MOE_LIB_PATH") or os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_SOFTMAX, MOE_SIGMOID = 0, 1
MOE_SWIGLU, MOE_GELU = 0, 1
MOE_GATE_TOPK, MOE_GATE_HASH = 0, 1
MOE_QUEUE_TOKEN, MOE_QUEUE_CHOICE = 0, 1
MOE_LOGITS_IN, MOE_LOGITS_OUT = 1, 2
MOE_FFN_GEMM1, MOE_FFN_GEMM2 = 1, 2
MOE_WS_LAYER, MOE_WS_ROUTE, MOE_WS_PERMUTE, MOE_WS_FFN, MOE_WS_BACKWARD = range(5)
INT32_MAX = 2**31 - 1


class MoeDesc(C.Structure):
    _fields_ = [
        ("T", C.c_int32), ("h", C.c_int32), ("H", C.c_int32), ("E", C.c_int32),
        ("K", C.c_int32), ("f", C.c_int32), ("n_shared", C.c_int32), ("has_wo", C.c_int32),
        ("dtype", C.c_int32), ("score", C.c_int32), ("act", C.c_int32),
        ("capacity_factor", C.c_float), ("aux_alpha", C.c_float),
        ("gate", C.c_int32), ("n_groups", C.c_int32), ("group_limit", C.c_int32), ("queue", C.c_int32),
        ("capacity_factor_eval", C.c_float), ("eval", C.c_int32), ("packed", C.c_int32),
    ]


class MoeWeights(C.Structure):
    _fields_ = [
        ("w_router", C.c_void_p), ("logit_bias", C.c_void_p), ("select_bias", C.c_void_p),
        ("w_gate", C.c_void_p), ("w_up", C.c_void_p), ("w_down", C.c_void_p),
        ("sh_gate", C.c_void_p), ("sh_up", C.c_void_p), ("sh_down", C.c_void_p),
        ("w_o", C.c_void_p), ("hash_keys", C.c_void_p),
    ]


class MoeAux(C.Structure):
    _fields_ = [
        ("topk_idx", C.c_void_p), ("topk_w", C.c_void_p), ("dest_row", C.c_void_p),
        ("counts", C.c_void_p), ("kept", C.c_void_p), ("n_kept", C.c_void_p),
        ("n_dropped", C.c_void_p), ("f", C.c_void_p), ("P", C.c_void_p), ("l_aux", C.c_void_p),
    ]


class MoeSaved(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("topk_idx", "topk_w", "dest_row", "src_token", "offsets", "counts",
                                          "logits", "act_grad", "h", "y_perm", "sh_act_grad", "sh_h", "y_cat")]


class MoeGrads(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("dx", "w_router", "w_gate", "w_up", "w_down", "sh_gate", "sh_up",
                                          "sh_down", "w_o")]


# exported symbol -> (restype, argtypes)
_VP = C.c_void_p
SIGNATURES = {
    "moe_capacity": (C.c_int32, [C.POINTER(MoeDesc)]),
    "moe_workspace_size": (C.c_int, [C.POINTER(MoeDesc), C.c_int32, C.POINTER(C.c_size_t)]),
    "moe_route": (C.c_int, [C.POINTER(MoeDesc), _VP, _VP, _VP, _VP, _VP, C.c_uint32, _VP, _VP, _VP, _VP,
                            _VP, C.c_size_t, _VP]),
    "moe_route_hash": (C.c_int, [C.POINTER(MoeDesc), _VP, _VP, _VP, _VP, _VP]),
    "moe_permute": (C.c_int, [C.POINTER(MoeDesc), _VP, _VP, C.c_int32, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                              _VP, C.c_size_t, _VP]),
    "moe_permute_noalloc": (C.c_int, [C.POINTER(MoeDesc), _VP, _VP, C.c_int32, _VP, _VP, _VP, _VP, _VP, _VP,
                                      _VP, _VP]),
    "moe_permute_noalloc_max_ints": (C.c_size_t, []),
    "moe_grouped_ffn": (C.c_int, [C.POINTER(MoeDesc), _VP, _VP, C.c_int32, _VP, _VP, _VP, _VP, _VP,
                                  C.c_uint32, _VP, C.c_size_t, _VP]),
    "moe_grouped_ffn_rows": (C.c_int, [C.POINTER(MoeDesc), _VP, _VP, _VP, C.c_int32, _VP, _VP, _VP, _VP, _VP,
                                       C.c_uint32, _VP, C.c_size_t, _VP]),
    "moe_combine": (C.c_int, [C.POINTER(MoeDesc), _VP, _VP, _VP, _VP, _VP, _VP]),
    "moe_pack_weights": (C.c_int, [_VP, _VP, C.c_int64, C.c_int32, C.c_int32, _VP]),
    "moe_layer_forward": (C.c_int, [C.POINTER(MoeDesc), C.POINTER(MoeWeights), _VP, _VP,
                                    C.POINTER(MoeAux), _VP, C.c_size_t, _VP]),
    "moe_max_rows": (C.c_int32, [C.POINTER(MoeDesc)]),
    "moe_layer_forward_train": (C.c_int, [C.POINTER(MoeDesc), C.POINTER(MoeWeights), _VP, _VP, C.POINTER(MoeAux),
                                          C.POINTER(MoeSaved), _VP, C.c_size_t, _VP]),
    "moe_layer_backward": (C.c_int, [C.POINTER(MoeDesc), C.POINTER(MoeWeights), _VP, _VP, C.POINTER(MoeSaved),
                                     C.c_float, C.POINTER(MoeGrads), _VP, C.c_size_t, _VP]),
    "moe_status_string": (C.c_char_p, [C.c_int]),
    "moe_last_error": (C.c_char_p, []),
    "moe_version": (C.c_char_p, []),
}

_lib = None


def lib():
    """The loaded libmoe.so; raises if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"libmoe.so not found at {LIB_PATH}: build it with "
                "`python -m mixture_experts_layer_45_amd.build` (hipcc, gfx950)")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib
