"""ctypes declarations of the C ABI in include/moe.h (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

from .build import LIB_PATH

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE, MOE_ERR_INTERNAL, \
    MOE_ERR_DATA = range(7)
MOE_DT_F32, MOE_DT_BF16 = 0, 1
MOE_W_MXFP4, MOE_W_RVQ3 = 0, 1
MOE_ACT_SWIGLU = 0
MOE_F_DETERMINISTIC = 1
MOE_ACT_SWIGLU, MOE_ACT_SITU = 0, 1
MOE_F_MX_GATEUP = 2
MOE_F_LORA = 4
MOE_F_QUANT_X8 = 8
MOE_F_VALIDATE = 16
MOE_F_RVQ_GATHER = 32
# bits of the MOE_F_VALIDATE status word
MOE_BAD_X, MOE_BAD_DY, MOE_BAD_SCALE_NAN, MOE_BAD_SCALE_ZERO, MOE_BAD_CODEWORD = 1, 2, 4, 8, 16

EXPORTED = (
    "moe_desc_init", "moe_workspace_size", "moe_layer_create", "moe_route", "moe_forward",
    "moe_backward_input", "moe_destroy", "moe_status_string", "moe_last_error",
    "moe_set_lora", "moe_backward_lora", "moe_check_status", "moe_forward_static",
    "moe_project_in", "moe_project_out", "moe_project_out_backward", "moe_project_in_backward", "moe_prof_enable", "moe_prof_read", "moe_prof_hbm_read",
)

# kernel families of include/moe_prof.h
PROF_ROUTER_LOGITS, PROF_ROUTER_TOPK, PROF_GROUP, PROF_GATEUP, PROF_DOWN, PROF_COMBINE, PROF_BWD_DOWN, \
    PROF_BWD_GATEUP, PROF_BWD_FINAL, PROF_XTERMS = range(10)
PROF_NAMES = ("router_logits", "router_topk", "group", "gateup", "down", "combine", "bwd_down", "bwd_gateup",
              "bwd_final", "xterms")


class MoeDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("inter", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("max_tokens", ctypes.c_int32), ("wfmt", ctypes.c_int32),
                ("act", ctypes.c_int32), ("bias_mode", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("n_shared", ctypes.c_int32), ("model_width", ctypes.c_int32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("router_w", ctypes.c_void_p), ("router_b", ctypes.c_void_p),
                ("codes", ctypes.c_void_p * 3), ("scales", ctypes.c_void_p * 3),
                ("rvq_idx", ctypes.c_void_p * 3), ("rvq_cb", ctypes.c_void_p * 3),
                ("shared_codes", ctypes.c_void_p * 3), ("shared_scales", ctypes.c_void_p * 3),
                ("shared_rvq_idx", ctypes.c_void_p * 3), ("shared_rvq_cb", ctypes.c_void_p * 3),
                ("proj_in", ctypes.c_void_p), ("proj_out", ctypes.c_void_p)]


class MoeLora(ctypes.Structure):
    _fields_ = [("rank", ctypes.c_int32), ("scale", ctypes.c_float), ("A", ctypes.c_void_p * 3),
                ("B", ctypes.c_void_p * 3)]


class MoeRouting(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("ids", "w", "counts", "offsets", "perm", "inv", "active", "n_active")]


class MoeError(RuntimeError):
    def __init__(self, status: int, fn: str, detail: str):
        super().__init__(f"{fn}: status {status} ({detail})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree gfx950 library; there is no other implementation to fall back to."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (quantized_moe_route_amd.build.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
        L.moe_desc_init.argtypes = [ctypes.POINTER(MoeDesc)]
        L.moe_desc_init.restype = None
        L.moe_workspace_size.argtypes = [ctypes.POINTER(MoeDesc), ctypes.POINTER(ctypes.c_size_t)]
        L.moe_workspace_size.restype = st
        L.moe_layer_create.argtypes = [ctypes.POINTER(MoeDesc), ctypes.POINTER(MoeWeights), vp, ctypes.c_size_t,
                                       ctypes.POINTER(vp)]
        L.moe_layer_create.restype = st
        L.moe_route.argtypes = [vp, vp, i32, i32, ctypes.POINTER(MoeRouting), vp]
        L.moe_route.restype = st
        L.moe_forward.argtypes = [vp, vp, i32, i32, ctypes.POINTER(MoeRouting), vp, vp, vp]
        L.moe_forward.restype = st
        L.moe_backward_input.argtypes = [vp, vp, i32, vp, i32, i32, ctypes.POINTER(MoeRouting), vp, vp, vp]
        L.moe_backward_input.restype = st
        L.moe_set_lora.argtypes = [vp, ctypes.POINTER(MoeLora)]
        L.moe_set_lora.restype = st
        L.moe_backward_lora.argtypes = [vp, vp, i32, vp, i32, i32, ctypes.POINTER(MoeRouting), vp, vp,
                                        ctypes.POINTER(vp), ctypes.POINTER(vp), vp]
        L.moe_backward_lora.restype = st
        L.moe_forward_static.argtypes = [vp, vp, i32, i32, ctypes.POINTER(MoeRouting), vp, vp]
        L.moe_forward_static.restype = st
        for fn in ("moe_project_in", "moe_project_out_backward"):
            getattr(L, fn).argtypes = [vp, vp, i32, i32, vp, vp]
            getattr(L, fn).restype = st
        for fn in ("moe_project_out", "moe_project_in_backward"):
            getattr(L, fn).argtypes = [vp, vp, i32, vp, vp]
            getattr(L, fn).restype = st
        L.moe_check_status.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32), vp]
        L.moe_check_status.restype = st
        L.moe_destroy.argtypes = [vp]
        L.moe_destroy.restype = None
        L.moe_status_string.argtypes = [st]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        L.moe_prof_enable.argtypes = [vp, ctypes.c_uint32, i32]
        L.moe_prof_enable.restype = st
        L.moe_prof_read.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i32)]
        L.moe_prof_read.restype = st
        L.moe_prof_hbm_read.argtypes = [vp, ctypes.c_size_t, vp, ctypes.POINTER(ctypes.c_double)]
        L.moe_prof_hbm_read.restype = st
        _lib = L
    return _lib


def check(status: int, fn: str) -> None:
    if status != MOE_OK:
        L = lib()
        raise MoeError(status, fn, (L.moe_last_error() or b"").decode() or L.moe_status_string(status).decode())
