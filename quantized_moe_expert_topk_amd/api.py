"""Python binding of the C ABI in ``include/qmoe.h``: the same entry points, taking torch
device tensors.  Argument marshalling only; every step runs in the gfx950 kernels of
``libqmoe.so``.  Output tensors are allocated with torch when the caller passes none.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import (MOE_FMT, MOE_LAYOUT_ROWS, MOE_LAYOUT_TILE16, MOE_OUT_BF16, MOE_OUT_F32, MoeAlignOutStruct,
                   MoeBankStruct, check, lib)



def _workspace(nbytes: int, device) -> torch.Tensor:
    """A device workspace.  With QMOE_POISON_WORKSPACE set (the test session sets it) every byte
    starts as 0xFF (e4m3 NaN, int32 -1), so that a kernel reading a byte nobody wrote shows up in
    its results instead of passing on leftovers of an earlier call."""
    ws = torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
    if os.environ.get("QMOE_POISON_WORKSPACE"):
        ws.fill_(0xFF)
    return ws

def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _need(t: torch.Tensor, dtype, shape, name):
    if t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous() or t.device.type != "cuda":
        raise ValueError(f"{name}: expected contiguous cuda {dtype} {tuple(shape)}, got {t.dtype} "
                         f"{tuple(t.shape)} on {t.device}")


@dataclass
class DeviceBank:
    """One bank of E experts on the GPU, in the full-I layout of ``moe_bank``; ``layout`` is
    MOE_LAYOUT_ROWS (the checkpoint's row-major order) or MOE_LAYOUT_TILE16 (the kernels' order,
    made once by :func:`moe_pack_bank`)."""
    fmt: str
    E: int
    H: int
    I: int
    gate_up: torch.Tensor
    gate_up_scale: torch.Tensor
    down: torch.Tensor
    down_scale: torch.Tensor
    gate_up_global: torch.Tensor | None = None
    down_global: torch.Tensor | None = None
    layout: int = MOE_LAYOUT_ROWS

    def struct(self) -> MoeBankStruct:
        return MoeBankStruct(MOE_FMT[self.fmt], self.E, self.H, self.I, self.gate_up.data_ptr(),
                             self.gate_up_scale.data_ptr(),
                             self.gate_up_global.data_ptr() if self.gate_up_global is not None else None,
                             self.down.data_ptr(), self.down_scale.data_ptr(),
                             self.down_global.data_ptr() if self.down_global is not None else None,
                             self.layout)

    def nbytes_expert(self) -> int:
        ts = [self.gate_up, self.gate_up_scale, self.down, self.down_scale, self.gate_up_global, self.down_global]
        return sum(t[0].numel() * t.element_size() for t in ts if t is not None)


@dataclass
class AlignOut:
    sorted_ids: torch.Tensor
    block_expert: torch.Tensor
    counts: torch.Tensor
    offsets: torch.Tensor
    total_padded: torch.Tensor
    block_m: int
    capacity: int

    def struct(self) -> MoeAlignOutStruct:
        return MoeAlignOutStruct(self.sorted_ids.data_ptr(), self.block_expert.data_ptr(), self.counts.data_ptr(),
                                 self.offsets.data_ptr(), self.total_padded.data_ptr(), self.block_m, self.capacity)


def moe_pack_bank(bank: DeviceBank, stream=None) -> DeviceBank:
    """The bank reordered into MOE_LAYOUT_TILE16 (new code and FP4 scale storage, in the
    row-major shapes; the FP8 block scales and NVFP4 globals are shared with ``bank``).  The
    source is row-major, or for MXFP4 also transposed (MOE_LAYOUT_MXFP4_T).  A packed bank is
    returned as is."""
    if bank.layout == MOE_LAYOUT_TILE16:
        return bank
    E, H, I = bank.E, bank.H, bank.I

    def like(t, rows, cols):  # new storage, [E, rows, cols] of t's dtype
        return torch.empty((E, rows, cols), dtype=t.dtype, device=t.device)

    if bank.fmt in ("nvfp4", "mxfp4", "q4_0"):  # codes and scales are reordered
        sdiv = 16 if bank.fmt == "nvfp4" else 32  # scale elements per row: K / sdiv
        gu, dn = like(bank.gate_up, 2 * I, H // 2), like(bank.down, H, I // 2)
        gus, dns = like(bank.gate_up_scale, 2 * I, H // sdiv), like(bank.down_scale, H, I // sdiv)
    else:  # codes only
        gu, dn = torch.empty_like(bank.gate_up), torch.empty_like(bank.down)
        gus, dns = bank.gate_up_scale, bank.down_scale
    dst = DeviceBank(bank.fmt, E, H, I, gu, gus, dn, dns, bank.gate_up_global, bank.down_global, MOE_LAYOUT_TILE16)
    src_s, dst_s = bank.struct(), dst.struct()
    check("moe_pack_bank", lib().moe_pack_bank(ctypes.byref(src_s), ctypes.byref(dst_s), _stream(stream)))
    return dst


# ----------------------------------------------------------------------------- routing

def moe_route_workspace_bytes(T: int, H: int, E: int) -> int:
    return int(lib().moe_route_workspace_bytes(T, H, E))


def moe_route(x: torch.Tensor, w_router: torch.Tensor, bias: torch.Tensor | None, k: int, renormalize: bool = True,
              logits=None, topk_ids=None, topk_w=None, workspace=None, stream=None):
    """Router logits, top-k ids and weights.  x [T,H] bf16, w_router [E,H] bf16, bias [E] f32."""
    T, H = x.shape
    E = w_router.shape[0]
    dev = x.device
    logits = torch.empty((T, E), dtype=torch.float32, device=dev) if logits is None else logits
    topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev) if topk_ids is None else topk_ids
    topk_w = torch.empty((T, k), dtype=torch.float32, device=dev) if topk_w is None else topk_w
    _need(x, torch.bfloat16, (T, H), "x")
    _need(w_router, torch.bfloat16, (E, H), "w_router")
    if bias is not None:
        _need(bias, torch.float32, (E,), "bias")
    _need(logits, torch.float32, (T, E), "logits")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    need = moe_route_workspace_bytes(T, H, E)
    if workspace is None and need:
        workspace = _workspace(need, dev)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    check("moe_route", lib().moe_route(_ptr(x), T, H, _ptr(w_router), E, _ptr(bias), k, int(renormalize),
                                       _ptr(logits), _ptr(topk_ids), _ptr(topk_w), _ptr(workspace), ws_bytes,
                                       _stream(stream)))
    return logits, topk_ids, topk_w


def moe_route_from_logits(logits: torch.Tensor, k: int, bias: torch.Tensor | None = None, renormalize: bool = True,
                          topk_ids=None, topk_w=None, stream=None):
    T, E = logits.shape
    dev = logits.device
    topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev) if topk_ids is None else topk_ids
    topk_w = torch.empty((T, k), dtype=torch.float32, device=dev) if topk_w is None else topk_w
    _need(logits, torch.float32, (T, E), "logits")
    if bias is not None:
        _need(bias, torch.float32, (E,), "bias")
    check("moe_route_from_logits", lib().moe_route_from_logits(_ptr(logits), T, E, _ptr(bias), k, int(renormalize),
                                                               _ptr(topk_ids), _ptr(topk_w), _stream(stream)))
    return topk_ids, topk_w


# ----------------------------------------------------------------------------- alignment

def moe_align_capacity(T: int, k: int, E: int, block_m: int) -> int:
    return int(lib().moe_align_capacity(T, k, E, block_m))


def moe_align_workspace_bytes(T: int, k: int, E: int) -> int:
    return int(lib().moe_align_workspace_bytes(T, k, E))


def alloc_align(T: int, k: int, E: int, block_m: int, device="cuda") -> AlignOut:
    cap = moe_align_capacity(T, k, E, block_m)
    if cap < 0:
        raise ValueError("bad alignment sizes")
    z = lambda n: torch.empty(max(n, 1), dtype=torch.int32, device=device)
    return AlignOut(z(cap), z(cap // block_m), z(E), z(E + 1), z(1), block_m, cap)


def moe_align(topk_ids: torch.Tensor, E: int, block_m: int, out: AlignOut | None = None,
              workspace: torch.Tensor | None = None, stream=None) -> AlignOut:
    T, k = topk_ids.shape
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    out = alloc_align(T, k, E, block_m, topk_ids.device) if out is None else out
    need = moe_align_workspace_bytes(T, k, E)
    if workspace is None and need:
        workspace = _workspace(need, topk_ids.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = out.struct()
    check("moe_align", lib().moe_align(_ptr(topk_ids), T, k, E, ctypes.byref(st), _ptr(workspace), ws_bytes,
                                       _stream(stream)))
    return out


def moe_route_align_workspace_bytes(T: int, H: int, E: int, k: int) -> int:
    return int(lib().moe_route_align_workspace_bytes(T, H, E, k))


def moe_route_align(x: torch.Tensor, w_router: torch.Tensor, bias: torch.Tensor | None, k: int, block_m: int,
                    renormalize: bool = True, logits=None, topk_ids=None, topk_w=None, out: AlignOut | None = None,
                    workspace=None, stream=None):
    """moe_route then moe_align in one call (one launch fewer for decode-sized batches).
    Returns (logits, topk_ids, topk_w, AlignOut)."""
    T, H = x.shape
    E = w_router.shape[0]
    dev = x.device
    logits = torch.empty((T, E), dtype=torch.float32, device=dev) if logits is None else logits
    topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev) if topk_ids is None else topk_ids
    topk_w = torch.empty((T, k), dtype=torch.float32, device=dev) if topk_w is None else topk_w
    _need(x, torch.bfloat16, (T, H), "x")
    _need(w_router, torch.bfloat16, (E, H), "w_router")
    if bias is not None:
        _need(bias, torch.float32, (E,), "bias")
    _need(logits, torch.float32, (T, E), "logits")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    out = alloc_align(T, k, E, block_m, dev) if out is None else out
    need = moe_route_align_workspace_bytes(T, H, E, k)
    if workspace is None and need:
        workspace = _workspace(need, dev)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = out.struct()
    check("moe_route_align", lib().moe_route_align(_ptr(x), T, H, _ptr(w_router), E, _ptr(bias), k, int(renormalize),
                                                   _ptr(logits), _ptr(topk_ids), _ptr(topk_w), ctypes.byref(st),
                                                   _ptr(workspace), ws_bytes, _stream(stream)))
    return logits, topk_ids, topk_w, out


# ----------------------------------------------------------------------------- expert layer

def moe_workspace_bytes(routed: DeviceBank, shared: DeviceBank | None, T: int, k: int, block_m: int,
                        slice_lo: int, slice_hi: int) -> int:
    rs = routed.struct()
    ss = shared.struct() if shared is not None else None
    return int(lib().moe_workspace_bytes(ctypes.byref(rs), ctypes.byref(ss) if ss is not None else None, T, k,
                                         block_m, slice_lo, slice_hi))


def _fwd_common(routed, shared, T, k, align, slice_lo, slice_hi, workspace, device):
    need = moe_workspace_bytes(routed, shared, T, k, align.block_m, slice_lo, slice_hi)
    if workspace is None:
        workspace = _workspace(need, device)
    rs, ss, al = routed.struct(), (shared.struct() if shared is not None else None), align.struct()
    return workspace, rs, ss, al


def moe_expert_forward(routed: DeviceBank, shared: DeviceBank | None, x: torch.Tensor, topk_w: torch.Tensor,
                       align: AlignOut, slice_lo: int, slice_hi: int, out=None, out_dtype=torch.float32,
                       workspace=None, stream=None) -> torch.Tensor:
    """This rank's [T, H] partial sum over the intermediate slice [slice_lo, slice_hi)."""
    T, H = x.shape
    k = topk_w.shape[1]
    _need(x, torch.bfloat16, (T, H), "x")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    out = torch.empty((T, H), dtype=out_dtype, device=x.device) if out is None else out
    _need(out, out_dtype, (T, H), "out")
    workspace, rs, ss, al = _fwd_common(routed, shared, T, k, align, slice_lo, slice_hi, workspace, x.device)
    code = MOE_OUT_BF16 if out_dtype == torch.bfloat16 else MOE_OUT_F32
    check("moe_expert_forward", lib().moe_expert_forward(
        ctypes.byref(rs), ctypes.byref(ss) if ss is not None else None, _ptr(x), T, k, _ptr(topk_w),
        ctypes.byref(al), slice_lo, slice_hi, _ptr(out), code, _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def moe_expert_forward_static(routed: DeviceBank, shared: DeviceBank | None, x: torch.Tensor, topk_w: torch.Tensor,
                              align: AlignOut, slice_lo: int, slice_hi: int, out: torch.Tensor, stream=None) -> torch.Tensor:
    """moe_expert_forward on the library's own fixed device scratch (no workspace argument);
    ``out`` must be passed (this call allocates nothing, here or in the library)."""
    T, H = x.shape
    k = topk_w.shape[1]
    _need(x, torch.bfloat16, (T, H), "x")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(out, out.dtype, (T, H), "out")
    rs, ss, al = routed.struct(), (shared.struct() if shared is not None else None), align.struct()
    code = MOE_OUT_BF16 if out.dtype == torch.bfloat16 else MOE_OUT_F32
    check("moe_expert_forward_static", lib().moe_expert_forward_static(
        ctypes.byref(rs), ctypes.byref(ss) if ss is not None else None, _ptr(x), T, k, _ptr(topk_w),
        ctypes.byref(al), slice_lo, slice_hi, _ptr(out), code, _stream(stream)))
    return out


def moe_expert_gate_up(routed: DeviceBank, shared: DeviceBank | None, x: torch.Tensor, k: int, align: AlignOut,
                       slice_lo: int, slice_hi: int, workspace: torch.Tensor, stream=None) -> None:
    T, H = x.shape
    _need(x, torch.bfloat16, (T, H), "x")
    workspace, rs, ss, al = _fwd_common(routed, shared, T, k, align, slice_lo, slice_hi, workspace, x.device)
    check("moe_expert_gate_up", lib().moe_expert_gate_up(
        ctypes.byref(rs), ctypes.byref(ss) if ss is not None else None, _ptr(x), T, k, ctypes.byref(al),
        slice_lo, slice_hi, _ptr(workspace), workspace.numel(), _stream(stream)))


def moe_expert_down(routed: DeviceBank, shared: DeviceBank | None, topk_w: torch.Tensor, align: AlignOut,
                    slice_lo: int, slice_hi: int, out: torch.Tensor, workspace: torch.Tensor, stream=None) -> None:
    T, k = topk_w.shape
    _need(topk_w, torch.float32, (T, k), "topk_w")
    workspace, rs, ss, al = _fwd_common(routed, shared, T, k, align, slice_lo, slice_hi, workspace, out.device)
    code = MOE_OUT_BF16 if out.dtype == torch.bfloat16 else MOE_OUT_F32
    check("moe_expert_down", lib().moe_expert_down(
        ctypes.byref(rs), ctypes.byref(ss) if ss is not None else None, T, k, _ptr(topk_w), ctypes.byref(al),
        slice_lo, slice_hi, _ptr(out), code, _ptr(workspace), workspace.numel(), _stream(stream)))


def moe_layer_forward(x: torch.Tensor, w_router: torch.Tensor, bias: torch.Tensor | None, k: int, renormalize: bool,
                      routed: DeviceBank, shared: DeviceBank | None, slice_lo: int, slice_hi: int,
                      logits: torch.Tensor, topk_ids: torch.Tensor, topk_w: torch.Tensor, align: AlignOut,
                      out: torch.Tensor, route_workspace: torch.Tensor | None, workspace: torch.Tensor,
                      stream=None) -> torch.Tensor:
    """The whole layer in one call (``moe_layer_forward``): moe_route_align then
    moe_expert_forward, with the same outputs; for one token the top-k and the alignment run
    inside the gate_up kernel."""
    T, H = x.shape
    E = w_router.shape[0]
    _need(x, torch.bfloat16, (T, H), "x")
    _need(w_router, torch.bfloat16, (E, H), "w_router")
    if bias is not None:
        _need(bias, torch.float32, (E,), "bias")
    _need(logits, torch.float32, (T, E), "logits")
    _need(topk_ids, torch.int32, (T, k), "topk_ids")
    _need(topk_w, torch.float32, (T, k), "topk_w")
    _need(out, out.dtype, (T, H), "out")
    rs, ss, al = routed.struct(), (shared.struct() if shared is not None else None), align.struct()
    code = MOE_OUT_BF16 if out.dtype == torch.bfloat16 else MOE_OUT_F32
    rws = route_workspace.numel() if route_workspace is not None else 0
    check("moe_layer_forward", lib().moe_layer_forward(
        _ptr(x), T, _ptr(w_router), _ptr(bias), k, int(renormalize), ctypes.byref(rs),
        ctypes.byref(ss) if ss is not None else None, slice_lo, slice_hi, _ptr(logits), _ptr(topk_ids),
        _ptr(topk_w), ctypes.byref(al), _ptr(out), code, _ptr(route_workspace), rws, _ptr(workspace),
        workspace.numel(), _stream(stream)))
    return out


def choose_block_m(T: int, k: int, E: int, fmt: str | None = None) -> int:
    """The library's block-size policy (``moe_choose_block_m``): 16 while experts see few
    tokens each, larger as the mean number of pairs per expert grows; 128 (the prefill GEMMs)
    once experts see enough tokens to reuse each weight tile, for the formats those kernels
    cover."""
    bm = int(lib().moe_choose_block_m(T, k, E, MOE_FMT.get(fmt, 0) if fmt else 0))
    if bm < 0:
        check("moe_choose_block_m", bm)
    return bm


class MoeLayer:
    """Pre-allocated buffers for one (bank, T, slice) and the call of one layer,
    moe_layer_forward (moe_route_align, then moe_expert_forward) on one stream, host-sync
    free, so it can be captured in a HIP graph.  Row-major banks are packed (moe_pack_bank) here, once; pass
    packed banks to share their storage between layers."""

    def __init__(self, routed: DeviceBank, shared: DeviceBank | None, w_router: torch.Tensor,
                 bias: torch.Tensor | None, T: int, k: int, slice_lo: int, slice_hi: int,
                 renormalize: bool = True, block_m: int | None = None, out_dtype=torch.float32):
        dev = w_router.device
        routed = moe_pack_bank(routed)
        shared = moe_pack_bank(shared) if shared is not None else None
        self.routed, self.shared, self.w_router, self.bias = routed, shared, w_router, bias
        self.T, self.k, self.lo, self.hi, self.renormalize = T, k, slice_lo, slice_hi, renormalize
        self.block_m = block_m or choose_block_m(T, k, routed.E, routed.fmt)
        E = routed.E
        self.logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        self.ids = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.align = alloc_align(T, k, E, self.block_m, dev)
        self.route_ws = _workspace(moe_route_align_workspace_bytes(T, routed.H, E, k), dev)
        self.ws = _workspace(moe_workspace_bytes(routed, shared, T, k, self.block_m, slice_lo, slice_hi), dev)
        self.out = torch.empty((T, routed.H), dtype=out_dtype, device=dev)

    def __call__(self, x: torch.Tensor, stream=None) -> torch.Tensor:
        return moe_layer_forward(x, self.w_router, self.bias, self.k, self.renormalize, self.routed, self.shared,
                                 self.lo, self.hi, self.logits, self.ids, self.w, self.align, self.out,
                                 self.route_ws, self.ws, stream)
