"""ctypes loader of ``libqmoe.so`` (the gfx950 HIP library).  Fails loudly when the
library has not been built; there is no fallback path."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqmoe.so")

MOE_OK = 0
MOE_ERR_INVALID_ARG = -1
MOE_ERR_ALIGNMENT = -2
MOE_ERR_UNSUPPORTED = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_HIP = -5

MOE_FMT = {"nvfp4": 1, "fp8blk": 2, "mxfp4": 3, "bf16": 4, "q4_0": 5}
MOE_OUT_F32, MOE_OUT_BF16 = 0, 1
MOE_STATIC_SCRATCH_BYTES = 64 << 20
MOE_LAYOUT_ROWS, MOE_LAYOUT_TILE16, MOE_LAYOUT_MXFP4_T = 0, 1, 2

# every entry point include/qmoe.h declares
EXPORTS = ("moe_route", "moe_route_workspace_bytes", "moe_route_from_logits", "moe_align_capacity",
           "moe_choose_block_m", "moe_align_workspace_bytes", "moe_align",
           "moe_route_align_workspace_bytes", "moe_route_align",
           "moe_workspace_bytes", "moe_pack_bank", "moe_expert_forward", "moe_expert_forward_static",
           "moe_expert_gate_up", "moe_expert_down", "moe_layer_forward",
           "moe_status_string", "moe_last_error")


class MoeBankStruct(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("gate_up", ctypes.c_void_p), ("gate_up_scale", ctypes.c_void_p),
                ("gate_up_global", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("down_scale", ctypes.c_void_p), ("down_global", ctypes.c_void_p), ("layout", ctypes.c_int32)]


class MoeAlignOutStruct(ctypes.Structure):
    _fields_ = [("sorted_ids", ctypes.c_void_p), ("block_expert", ctypes.c_void_p), ("counts", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p), ("total_padded", ctypes.c_void_p), ("block_m", ctypes.c_int32),
                ("capacity", ctypes.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, name: str, status: int, detail: str):
        super().__init__(f"{name} failed with status {status}: {detail}")
        self.status = status
        self.detail = detail


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library.  Raises if it is missing (build with
    ``python -m quantized_moe_expert_topk_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: the gfx950 HIP library must be built first "
                              "(python -m quantized_moe_expert_topk_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        i32, vp, sz = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        pb = ctypes.POINTER(MoeBankStruct)
        pa = ctypes.POINTER(MoeAlignOutStruct)
        L.moe_route.argtypes = [vp, i32, i32, vp, i32, vp, i32, i32, vp, vp, vp, vp, sz, vp]
        L.moe_route_workspace_bytes.argtypes = [i32, i32, i32]
        L.moe_route_workspace_bytes.restype = sz
        L.moe_route_from_logits.argtypes = [vp, i32, i32, vp, i32, i32, vp, vp, vp]
        L.moe_align_capacity.argtypes = [i32, i32, i32, i32]
        L.moe_align_capacity.restype = ctypes.c_int32
        L.moe_choose_block_m.argtypes = [i32, i32, i32, i32]
        L.moe_choose_block_m.restype = ctypes.c_int32
        L.moe_align_workspace_bytes.argtypes = [i32, i32, i32]
        L.moe_align_workspace_bytes.restype = sz
        L.moe_align.argtypes = [vp, i32, i32, i32, pa, vp, sz, vp]
        L.moe_route_align_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.moe_route_align_workspace_bytes.restype = sz
        L.moe_route_align.argtypes = [vp, i32, i32, vp, i32, vp, i32, i32, vp, vp, vp, pa, vp, sz, vp]
        L.moe_workspace_bytes.argtypes = [pb, pb, i32, i32, i32, i32, i32]
        L.moe_workspace_bytes.restype = sz
        L.moe_pack_bank.argtypes = [pb, pb, vp]
        L.moe_expert_forward.argtypes = [pb, pb, vp, i32, i32, vp, pa, i32, i32, vp, i32, vp, sz, vp]
        L.moe_expert_forward_static.argtypes = [pb, pb, vp, i32, i32, vp, pa, i32, i32, vp, i32, vp]
        L.moe_expert_gate_up.argtypes = [pb, pb, vp, i32, i32, pa, i32, i32, vp, sz, vp]
        L.moe_expert_down.argtypes = [pb, pb, i32, i32, vp, pa, i32, i32, vp, i32, vp, sz, vp]
        L.moe_layer_forward.argtypes = [vp, i32, vp, vp, i32, i32, pb, pb, i32, i32, vp, vp, vp, pa, vp, i32, vp, sz,
                                        vp, sz, vp]
        L.moe_status_string.argtypes = [i32]
        L.moe_status_string.restype = ctypes.c_char_p
        L.moe_last_error.argtypes = []
        L.moe_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def check(name: str, rc: int) -> None:
    if rc != MOE_OK:
        raise MoeError(name, rc, lib().moe_last_error().decode())
