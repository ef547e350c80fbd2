"""ctypes front-end of the fp64 CPU oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py``; never by the product package.  Arrays cross the boundary
as numpy buffers; nothing here touches a GPU.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

FMT = {"nvfp4": 1, "fp8blk": 2, "mxfp4": 3, "bf16": 4, "q4_0": 5}


def build(force: bool = False) -> str:
    """Compile ``liboracle.so`` (plain C, gcc -O2, no fast-math, OpenMP)."""
    src = os.path.join(_HERE, "oracle.c")
    hdr = os.path.join(_HERE, "oracle.h")
    newest = max(os.path.getmtime(src), os.path.getmtime(hdr))
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < newest:
        cmd = f"gcc -O2 -fno-fast-math -fopenmp -fPIC -shared -o {_LIB_PATH}.tmp {src} -lm && mv {_LIB_PATH}.tmp {_LIB_PATH}"
        if os.system(cmd) != 0:
            raise RuntimeError(f"oracle build failed: {cmd}")
    return _LIB_PATH


class _Bank(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int), ("E", ctypes.c_int), ("H", ctypes.c_int), ("I", ctypes.c_int),
                ("gate_up", ctypes.c_void_p), ("gate_up_scale", ctypes.c_void_p),
                ("gate_up_global", ctypes.c_void_p), ("down", ctypes.c_void_p),
                ("down_scale", ctypes.c_void_p), ("down_global", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32, u32, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_double
        for name in ("oracle_e2m1", "oracle_e4m3fn", "oracle_e8m0", "oracle_bf16", "oracle_f16"):
            getattr(L, name).restype = dbl
            getattr(L, name).argtypes = [u32]
        pb = ctypes.POINTER(_Bank)
        L.oracle_weight_gate_up.restype = dbl
        L.oracle_weight_gate_up.argtypes = [pb, i32, i32, i32]
        L.oracle_weight_down.restype = dbl
        L.oracle_weight_down.argtypes = [pb, i32, i32, i32]
        L.oracle_router_logits.argtypes = [vp, i32, i32, vp, i32, vp, vp]
        L.oracle_topk.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp]
        L.oracle_route.argtypes = [vp, i32, i32, vp, i32, vp, i32, i32, vp, vp, vp, vp]
        L.oracle_align_capacity.restype = ctypes.c_int32
        L.oracle_align_capacity.argtypes = [i32, i32, i32, i32]
        L.oracle_align.argtypes = [vp, i32, i32, i32, i32, vp, vp, vp, vp, vp]
        L.oracle_expert_forward.argtypes = [pb, pb, vp, i32, i32, vp, vp, i32, i32, vp]
        L.oracle_dequant_gate_up.argtypes = [pb, i32, vp]
        L.oracle_dequant_down.argtypes = [pb, i32, vp]
        L.oracle_num_threads.restype = i32
        L.oracle_num_threads.argtypes = []
        _lib = L
    return _lib


def _p(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle takes C-contiguous arrays"
    return ctypes.c_void_p(a.ctypes.data)


def bank_struct(bank) -> _Bank:
    """Wrap a ``synth.Bank``-like object (attributes fmt,E,H,I and the six arrays)."""
    s = _Bank(FMT[bank.fmt], bank.E, bank.H, bank.I, _p(bank.gate_up), _p(bank.gate_up_scale),
              _p(bank.gate_up_global), _p(bank.down), _p(bank.down_scale), _p(bank.down_global))
    s._keep = bank  # keep the arrays alive
    return s


# ----------------------------------------------------------------------------- scalars

def num_threads() -> int:
    return int(lib().oracle_num_threads())


def e2m1(code: int) -> float:
    return lib().oracle_e2m1(code)


def e4m3fn(b: int) -> float:
    return lib().oracle_e4m3fn(b)


def e8m0(b: int) -> float:
    return lib().oracle_e8m0(b)


def bf16(bits: int) -> float:
    return lib().oracle_bf16(bits)


def f16(bits: int) -> float:
    return lib().oracle_f16(bits)


def weight_gate_up(bank, e, r, c) -> float:
    return lib().oracle_weight_gate_up(ctypes.byref(bank_struct(bank)), e, r, c)


def weight_down(bank, e, n, i) -> float:
    return lib().oracle_weight_down(ctypes.byref(bank_struct(bank)), e, n, i)


def dequant_gate_up(bank, e) -> np.ndarray:
    out = np.empty((2 * bank.I, bank.H), np.float64)
    lib().oracle_dequant_gate_up(ctypes.byref(bank_struct(bank)), e, _p(out))
    return out


def dequant_down(bank, e) -> np.ndarray:
    out = np.empty((bank.H, bank.I), np.float64)
    lib().oracle_dequant_down(ctypes.byref(bank_struct(bank)), e, _p(out))
    return out


# ----------------------------------------------------------------------------- routing

def router_logits(x: np.ndarray, wr: np.ndarray, bias=None) -> np.ndarray:
    T, H = x.shape
    E = wr.shape[0]
    out = np.empty((T, E), np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    lib().oracle_router_logits(_p(np.ascontiguousarray(x)), T, H, _p(np.ascontiguousarray(wr)), E, _p(b), _p(out))
    return out


def topk(score: np.ndarray, k: int, renormalize: bool = True):
    score = np.ascontiguousarray(score, np.float64)
    T, E = score.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    gap = np.empty(T, np.float64)
    rc = lib().oracle_topk(_p(score), T, E, k, int(renormalize), _p(ids), _p(w), _p(gap))
    if rc:
        raise ValueError(f"oracle_topk rc={rc}")
    return ids, w, gap


def route(x, wr, bias, k: int, renormalize: bool = True):
    """Returns (logits fp64 [T,E], ids [T,k], w fp64 [T,k], gap [T]).  Selection and weights
    are taken on the fp32-rounded logits; ``gap`` is in those fp32 values."""
    T, H = x.shape
    E = wr.shape[0]
    lg = np.empty((T, E), np.float64)
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float64)
    gap = np.empty(T, np.float64)
    b = None if bias is None else np.ascontiguousarray(bias, np.float32)
    rc = lib().oracle_route(_p(np.ascontiguousarray(x)), T, H, _p(np.ascontiguousarray(wr)), E, _p(b), k,
                            int(renormalize), _p(lg), _p(ids), _p(w), _p(gap))
    if rc:
        raise ValueError(f"oracle_route rc={rc}")
    return lg, ids, w, gap


# ----------------------------------------------------------------------------- align

def align_capacity(T: int, k: int, E: int, BM: int) -> int:
    return int(lib().oracle_align_capacity(T, k, E, BM))


def align(ids: np.ndarray, E: int, BM: int) -> dict:
    ids = np.ascontiguousarray(ids, np.int32)
    T, k = ids.shape
    cap = align_capacity(T, k, E, BM)
    out = dict(sorted_ids=np.empty(cap, np.int32), block_expert=np.empty(cap // BM, np.int32),
               counts=np.empty(E, np.int32), offsets=np.empty(E + 1, np.int32),
               total_padded=np.empty(1, np.int32))
    rc = lib().oracle_align(_p(ids), T, k, E, BM, _p(out["sorted_ids"]), _p(out["block_expert"]),
                            _p(out["counts"]), _p(out["offsets"]), _p(out["total_padded"]))
    if rc:
        raise ValueError(f"oracle_align rc={rc}")
    return out


# ----------------------------------------------------------------------------- expert layer

def expert_forward(routed, shared, x: np.ndarray, ids: np.ndarray, w: np.ndarray, lo: int, hi: int) -> np.ndarray:
    x = np.ascontiguousarray(x)
    ids = np.ascontiguousarray(ids, np.int32)
    w = np.ascontiguousarray(w, np.float64)
    T, k = ids.shape
    out = np.empty((T, routed.H), np.float64)
    rb = bank_struct(routed)
    sb = bank_struct(shared) if shared is not None else None
    rc = lib().oracle_expert_forward(ctypes.byref(rb), ctypes.byref(sb) if sb is not None else None,
                                     _p(x), T, k, _p(ids), _p(w), lo, hi, _p(out))
    if rc:
        raise ValueError(f"oracle_expert_forward rc={rc}")
    return out


def layer(inputs, T_rows=None, lo=0, hi=None):
    """Whole oracle layer on ``synth.LayerInputs``: route, then the expert forward.
    Returns dict(logits, ids, w, gap, out)."""
    cfg = inputs.cfg
    hi = cfg.I if hi is None else hi
    x = inputs.x if T_rows is None else np.ascontiguousarray(inputs.x[T_rows])
    lg, ids, w, gap = route(x, inputs.router, inputs.bias, cfg.k, cfg.renormalize)
    out = expert_forward(inputs.routed, inputs.shared, x, ids, w, lo, hi)
    return dict(logits=lg, ids=ids, w=w, gap=gap, out=out)
