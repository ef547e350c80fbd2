"""Host-side checks of the C ABI (CPU only): the library loads, exports every entry point
include/qmoe.h declares, and rejects bad arguments with the documented codes before it
touches a device.  No call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

import quantized_moe_expert_topk_amd as qm
from quantized_moe_expert_topk_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # a non-NULL pointer value; validation never dereferences it


def _header_functions():
    src = open(os.path.join(ROOT, "include", "qmoe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_entry_point():
    names = _header_functions()
    assert set(names) == set(L.EXPORTS), names
    lib = L.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = L.lib()
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.moe_status_string(code)
    assert lib.moe_status_string(-99) == b"unknown status"


def test_align_capacity_and_workspace_sizes():
    assert qm.moe_align_capacity(16, 2, 8, 16) == 32 + 8 * 15 + 8  # 160 rounded up to 16 -> 160
    for T, k, E, bm in [(1, 8, 256, 16), (64, 8, 256, 16), (8192, 8, 256, 64), (0, 8, 256, 16)]:
        c = qm.moe_align_capacity(T, k, E, bm)
        assert c % bm == 0 and c >= T * k + E * (bm - 1) and c - (T * k + E * (bm - 1)) < bm
    assert qm.moe_align_capacity(-1, 8, 256, 16) == -1
    assert qm.moe_align_workspace_bytes(8192, 8, 256) == 64 * 256 * 4
    assert qm.moe_align_workspace_bytes(0, 8, 256) == 0


@pytest.mark.parametrize("T,k,E,fmt,bm", [
    (1, 8, 256, "nvfp4", 16), (64, 8, 256, "nvfp4", 16), (512, 8, 256, "nvfp4", 16),   # <= 16 pairs/expert
    (513, 8, 256, "nvfp4", 32), (1023, 8, 256, "nvfp4", 32),                         # (16, 32)
    (1024, 8, 256, "nvfp4", 128), (8192, 8, 256, "nvfp4", 128), (4096, 8, 256, "fp8blk", 128),
    (8192, 8, 256, "bf16", 128),                                                       # >= 32: prefill GEMMs
    (1024, 8, 256, "mxfp4", 32), (2048, 8, 256, "mxfp4", 32), (2049, 8, 256, "mxfp4", 64),
    (8192, 8, 256, "q4_0", 64), (1024, 8, 256, None, 32), (16, 2, 8, "nvfp4", 16), (0, 8, 256, "nvfp4", 16),
])
def test_choose_block_m_policy(T, k, E, fmt, bm):
    """The library's block-size policy, through the C ABI: pairs per expert on average against
    16, 32 and 64, and the prefill GEMMs (128) only for the formats they cover."""
    assert qm.choose_block_m(T, k, E, fmt) == bm
    assert L.lib().moe_choose_block_m(T, k, E, L.MOE_FMT.get(fmt, 0) if fmt else 0) == bm


def test_choose_block_m_rejects_bad_sizes():
    lib = L.lib()
    for args in ((-1, 8, 256, 1), (4, 0, 256, 1), (4, 8, 0, 1)):
        assert lib.moe_choose_block_m(*args) == L.MOE_ERR_INVALID_ARG
        assert lib.moe_last_error()


def _bank(fmt=1, E=8, H=256, I=128, glob=True, layout=L.MOE_LAYOUT_TILE16, base=FAKE):
    return L.MoeBankStruct(fmt, E, H, I, base, base, base if glob else None, base, base, base if glob else None,
                           layout)


def _align(bm=16, cap=None, T=16, k=2, E=8):
    cap = qm.moe_align_capacity(T, k, E, bm) if cap is None else cap
    return L.MoeAlignOutStruct(FAKE, FAKE, FAKE, FAKE, FAKE, bm, cap)


def _fwd(bank=None, shared=None, T=16, k=2, lo=0, hi=128, al=None, ws=1 << 30, out_dtype=0, x=FAKE):
    lib = L.lib()
    bank = bank or _bank()
    al = al or _align(T=T, k=k, E=bank.E)
    rc = lib.moe_expert_forward(ctypes.byref(bank), ctypes.byref(shared) if shared else None, x, T, k, FAKE,
                                ctypes.byref(al), lo, hi, FAKE, out_dtype, FAKE, ws, None)
    return rc, lib.moe_last_error().decode()


FORWARD_REJECTS = [
    (dict(lo=8, hi=128), L.MOE_ERR_ALIGNMENT),                 # NVFP4 block is 16
    (dict(lo=64, hi=64), L.MOE_ERR_ALIGNMENT),                 # empty slice
    (dict(lo=0, hi=144), L.MOE_ERR_ALIGNMENT),                 # past I
    (dict(lo=-16, hi=64), L.MOE_ERR_ALIGNMENT),
    (dict(lo=16, hi=128), L.MOE_ERR_UNSUPPORTED),              # 16-aligned but the kernels need 32
    (dict(k=0), L.MOE_ERR_INVALID_ARG),
    (dict(k=9), L.MOE_ERR_INVALID_ARG),                        # k > E
    (dict(T=-1), L.MOE_ERR_INVALID_ARG),
    (dict(ws=100), L.MOE_ERR_WORKSPACE),
    (dict(bank=_bank(fmt=7)), L.MOE_ERR_INVALID_ARG),
    (dict(bank=_bank(glob=False)), L.MOE_ERR_INVALID_ARG),     # NVFP4 needs globals
    (dict(bank=_bank(H=200)), L.MOE_ERR_UNSUPPORTED),
    (dict(bank=_bank(fmt=2, I=192), hi=128), L.MOE_ERR_ALIGNMENT),  # fp8-block I % 128
    (dict(bank=_bank(fmt=2, I=256), lo=64, hi=192), L.MOE_ERR_ALIGNMENT),  # fp8-block slice % 128
    (dict(bank=_bank(fmt=3), lo=16, hi=128), L.MOE_ERR_ALIGNMENT),  # MXFP4 block is 32
    (dict(bank=_bank(fmt=5, glob=False, I=256), lo=16, hi=128), L.MOE_ERR_ALIGNMENT),  # Q4_0 block is 32
    (dict(bank=_bank(fmt=5, glob=False, I=96), hi=96), L.MOE_ERR_UNSUPPORTED),  # Q4_0 bank I % 128
    (dict(al=_align(bm=8)), L.MOE_ERR_UNSUPPORTED),
    (dict(al=_align(cap=32)), L.MOE_ERR_INVALID_ARG),
    (dict(shared=_bank(E=2)), L.MOE_ERR_INVALID_ARG),          # shared must be one expert
    (dict(shared=_bank(E=1, I=64)), L.MOE_ERR_INVALID_ARG),    # and the same I
    (dict(out_dtype=5), L.MOE_ERR_INVALID_ARG),
    (dict(x=None), L.MOE_ERR_INVALID_ARG),
    (dict(bank=_bank(layout=L.MOE_LAYOUT_ROWS)), L.MOE_ERR_UNSUPPORTED),  # kernels read TILE16 banks
    (dict(shared=_bank(E=1, layout=L.MOE_LAYOUT_ROWS)), L.MOE_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("kw,code", FORWARD_REJECTS)
def test_forward_rejects_bad_arguments_before_any_launch(kw, code):
    rc, msg = _fwd(**kw)
    assert rc == code, (rc, msg)
    assert msg


def _layer(bank=None, shared=None, T=16, k=2, lo=0, hi=128, al=None, ws=1 << 30, out_dtype=0, x=FAKE, wr=FAKE,
           rws=1 << 30, routed_null=False, ws_ptr=FAKE + (1 << 31)):
    lib = L.lib()
    bank = bank or _bank()
    al = al or _align(T=T, k=k, E=bank.E)
    rc = lib.moe_layer_forward(x, T, wr, None, k, 1, None if routed_null else ctypes.byref(bank),
                               ctypes.byref(shared) if shared else None, lo, hi, FAKE, FAKE, FAKE, ctypes.byref(al),
                               FAKE, out_dtype, FAKE, rws, ws_ptr, ws, None)
    return rc, lib.moe_last_error().decode()


@pytest.mark.parametrize("kw,code", FORWARD_REJECTS + [
    (dict(wr=None), L.MOE_ERR_INVALID_ARG),                    # the router weight
    (dict(rws=0), L.MOE_ERR_WORKSPACE),                        # the router's split-K partials
    (dict(routed_null=True), L.MOE_ERR_INVALID_ARG),
    (dict(bank=_bank(E=2048, I=128), k=2), L.MOE_ERR_UNSUPPORTED),  # the router needs E <= 1024
    (dict(bank=_bank(E=128), k=65), L.MOE_ERR_UNSUPPORTED),          # and k <= 64
    (dict(ws_ptr=FAKE + 64), L.MOE_ERR_INVALID_ARG),                # the two workspaces overlap
])
def test_layer_forward_rejects_bad_arguments_before_any_launch(kw, code):
    """moe_layer_forward runs the checks of moe_route_align and moe_expert_forward: the same
    codes for the forward's bad arguments, and the router's own."""
    rc, msg = _layer(**kw)
    assert rc == code, (rc, msg)
    assert msg


def test_route_and_align_reject_bad_arguments():
    lib = L.lib()
    W = 1 << 30
    assert lib.moe_route(None, 4, 256, FAKE, 8, None, 2, 1, FAKE, FAKE, FAKE, FAKE, W, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_route(FAKE, 4, 256, FAKE, 8, None, 9, 1, FAKE, FAKE, FAKE, FAKE, W, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_route(FAKE, 4, 200, FAKE, 8, None, 2, 1, FAKE, FAKE, FAKE, FAKE, W, None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_route(FAKE, 4, 256, FAKE, 2048, None, 2, 1, FAKE, FAKE, FAKE, FAKE, W, None) == L.MOE_ERR_UNSUPPORTED
    assert lib.moe_route_workspace_bytes(64, 2048, 256) > 0
    assert lib.moe_route(FAKE, 64, 2048, FAKE, 256, None, 8, 1, FAKE, FAKE, FAKE, FAKE, 0, None) == L.MOE_ERR_WORKSPACE
    assert lib.moe_route_from_logits(FAKE, 4, 8, None, 0, 1, FAKE, FAKE, None) == L.MOE_ERR_INVALID_ARG
    al = _align(T=16, k=2, E=8)
    assert lib.moe_align(FAKE, 16, 2, 8, ctypes.byref(al), FAKE, 0, None) == L.MOE_ERR_WORKSPACE
    assert lib.moe_align(None, 16, 2, 8, ctypes.byref(al), FAKE, 1 << 20, None) == L.MOE_ERR_INVALID_ARG
    small = _align(cap=16)
    assert lib.moe_align(FAKE, 16, 2, 8, ctypes.byref(small), FAKE, 1 << 20, None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_align(FAKE, 16, 2, 2048, ctypes.byref(al), FAKE, 1 << 20, None) == L.MOE_ERR_UNSUPPORTED


def test_route_align_rejects_bad_arguments():
    lib = L.lib()
    W = 1 << 30
    al = _align(T=16, k=2, E=8)
    ra = lib.moe_route_align
    assert ra(None, 16, 256, FAKE, 8, None, 2, 1, FAKE, FAKE, FAKE, ctypes.byref(al), FAKE, W, None) == L.MOE_ERR_INVALID_ARG
    assert ra(FAKE, 16, 256, FAKE, 8, None, 9, 1, FAKE, FAKE, FAKE, ctypes.byref(al), FAKE, W, None) == L.MOE_ERR_INVALID_ARG
    assert ra(FAKE, 16, 200, FAKE, 8, None, 2, 1, FAKE, FAKE, FAKE, ctypes.byref(al), FAKE, W, None) == L.MOE_ERR_UNSUPPORTED
    small = _align(cap=16)
    assert ra(FAKE, 16, 256, FAKE, 8, None, 2, 1, FAKE, FAKE, FAKE, ctypes.byref(small), FAKE, W, None) == L.MOE_ERR_INVALID_ARG
    assert ra(FAKE, 16, 256, FAKE, 8, None, 2, 1, FAKE, FAKE, FAKE, None, FAKE, W, None) == L.MOE_ERR_INVALID_ARG
    need = lib.moe_route_align_workspace_bytes(16, 256, 8, 2)
    assert need >= lib.moe_route_workspace_bytes(16, 256, 8) + lib.moe_align_workspace_bytes(16, 2, 8)
    assert ra(FAKE, 16, 256, FAKE, 8, None, 2, 1, FAKE, FAKE, FAKE, ctypes.byref(al), FAKE, need - 1, None) == L.MOE_ERR_WORKSPACE


def test_workspace_bytes_formula():
    b = _bank(E=8, H=256, I=128)
    s = _bank(E=1, H=256, I=128)
    lib = L.lib()
    T, k, bm = 16, 2, 16
    cap = qm.moe_align_capacity(T, k, 8, bm)
    h = -(-((cap + 128) * 64 * 2) // 256) * 256
    y = -(-((T * k + T) * 256 * 4) // 256) * 256
    assert lib.moe_workspace_bytes(ctypes.byref(b), ctypes.byref(s), T, k, bm, 0, 64) == h + y
    # MXFP4: the intermediate and the activation as two e4m3 planes plus their e8m0 scales
    mb, ms = _bank(fmt=3, glob=False), _bank(fmt=3, E=1, glob=False)
    up = lambda n: -(-n // 256) * 256  # noqa: E731
    rows = cap + 128
    want = up(2 * rows * 64) + up(2 * rows * 2) + up(2 * T * 256) + up(2 * T * 8) + y
    assert lib.moe_workspace_bytes(ctypes.byref(mb), ctypes.byref(ms), T, k, bm, 0, 64) == want


def _pack(src, dst):
    rc = L.lib().moe_pack_bank(ctypes.byref(src) if src else None, ctypes.byref(dst) if dst else None, None)
    return rc, L.lib().moe_last_error().decode()


@pytest.mark.parametrize("src,dst,code", [
    (None, _bank(), L.MOE_ERR_INVALID_ARG),
    (_bank(layout=L.MOE_LAYOUT_TILE16), _bank(base=0x40000000), L.MOE_ERR_INVALID_ARG),   # src must be ROWS
    (_bank(layout=L.MOE_LAYOUT_ROWS), _bank(layout=L.MOE_LAYOUT_ROWS, base=0x40000000), L.MOE_ERR_INVALID_ARG),
    (_bank(layout=L.MOE_LAYOUT_ROWS), _bank(I=256, base=0x40000000), L.MOE_ERR_INVALID_ARG),  # shape differs
    (_bank(layout=L.MOE_LAYOUT_ROWS), _bank(), L.MOE_ERR_INVALID_ARG),                    # dst overlaps src
    (_bank(layout=L.MOE_LAYOUT_ROWS, base=0x10008), _bank(base=0x40000000), L.MOE_ERR_INVALID_ARG),  # unaligned
    (_bank(layout=L.MOE_LAYOUT_ROWS, glob=False), _bank(base=0x40000000, glob=False), L.MOE_ERR_INVALID_ARG),
    (_bank(layout=L.MOE_LAYOUT_ROWS, I=48), _bank(I=48, base=0x40000000), L.MOE_ERR_UNSUPPORTED),  # half pieces
    (_bank(fmt=9, layout=L.MOE_LAYOUT_ROWS), _bank(fmt=9, base=0x40000000), L.MOE_ERR_INVALID_ARG),
    (_bank(fmt=1, layout=L.MOE_LAYOUT_MXFP4_T), _bank(base=0x40000000), L.MOE_ERR_INVALID_ARG),  # NVFP4 transposed
    (_bank(fmt=5, glob=False, I=64, layout=L.MOE_LAYOUT_ROWS), _bank(fmt=5, glob=False, I=64, base=0x40000000),
     L.MOE_ERR_UNSUPPORTED),  # Q4_0 pieces hold 4 whole blocks: I % 128
])
def test_pack_bank_rejects_bad_arguments_before_any_launch(src, dst, code):
    rc, msg = _pack(src, dst)
    assert rc == code, (rc, msg)
    assert msg



def test_forward_static_rejects_before_any_launch():
    """moe_expert_forward_static checks its arguments like moe_expert_forward, and a call whose
    workspace exceeds the library's fixed scratch fails with MOE_ERR_WORKSPACE, all before it
    touches a device."""
    lib = L.lib()
    b = _bank(E=256, H=2048, I=512)
    T, k, bm = 8192, 8, 128
    al = _align(bm=bm, T=T, k=k, E=256)
    assert lib.moe_workspace_bytes(ctypes.byref(b), None, T, k, bm, 0, 512) > L.MOE_STATIC_SCRATCH_BYTES
    rc = lib.moe_expert_forward_static(ctypes.byref(b), None, FAKE, T, k, FAKE, ctypes.byref(al), 0, 512, FAKE, 0,
                                       None)
    assert rc == L.MOE_ERR_WORKSPACE and b"scratch" in lib.moe_last_error()
    small = _align(T=16, k=2, E=8)
    bad = _bank()
    assert lib.moe_expert_forward_static(ctypes.byref(bad), None, FAKE, 16, 2, FAKE, ctypes.byref(small), 8, 128,
                                         FAKE, 0, None) == L.MOE_ERR_ALIGNMENT
    assert lib.moe_expert_forward_static(None, None, FAKE, 16, 2, FAKE, ctypes.byref(small), 0, 128, FAKE, 0,
                                         None) == L.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_forward_static(ctypes.byref(bad), None, FAKE, 16, 2, FAKE, ctypes.byref(small), 0, 128,
                                         FAKE, 7, None) == L.MOE_ERR_INVALID_ARG
