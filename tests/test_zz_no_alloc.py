"""moe_expert_forward_static -- the forward pass on the library's own fixed device scratch,
for callers that cannot allocate -- against moe_expert_forward with a caller workspace, on
consecutive calls (the second one smaller, so it runs over what the first left in the
scratch), for both kernel families."""
import ctypes

import numpy as np
import pytest
import torch

import quantized_moe_expert_topk_amd as qm
from quantized_moe_expert_topk_amd import _lib as L
from oracle import oracle as O
from synth import synth as S
from tests.gpu_util import bf16_dev, check_close, device_bank, to_dev

pytestmark = pytest.mark.gpu


def _case(cid, T, lo, hi, bm=None, seed_batch=0):
    cfg = S.CONFIGS[cid]
    base = S.layer_inputs(cfg, T, batch=seed_batch, experts=[])
    _, ids, w, _ = O.route(base.x, base.router, base.bias, cfg.k, cfg.renormalize)
    inp = S.layer_inputs(cfg, T, batch=seed_batch, experts=np.unique(ids))
    bm = bm or qm.choose_block_m(T, cfg.k, cfg.E, cfg.fmt)
    rb = device_bank(inp.routed)
    sb = device_bank(inp.shared) if inp.shared is not None else None
    al = qm.moe_align(to_dev(ids.astype(np.int32)), cfg.E, bm)
    return inp, ids, w, rb, sb, al, bm


@pytest.mark.parametrize("first,second", [
    ((2, 64, 0, 512, None), (2, 8, 0, 256, None)),          # NVFP4 streaming, then a smaller batch and slice
    ((5, 256, 0, 1024, None), (5, 16, 1024, 2048, None)),   # MXFP4 planes, the largest decode workload
    ((2, 512, 0, 256, 128), (2, 300, 256, 512, 128)),       # the prefill GEMMs (align blocks of 128)
    ((4, 64, 0, 512, None), (7, 3, 96, 224, None)),         # fp8-block, then q4_0 on another bank
])
def test_static_scratch_forward_matches_caller_workspace(first, second):
    torch.cuda.synchronize()
    for n, (cid, T, lo, hi, bm) in enumerate((first, second)):
        inp, ids, w, rb, sb, al, bm = _case(cid, T, lo, hi, bm)
        x, wd = bf16_dev(inp.x), to_dev(w.astype(np.float32))
        name = f"call {n + 1}: cfg{cid} T={T} [{lo},{hi}) bm={bm}"
        print(f"[static] {name}", flush=True)
        need = qm.moe_workspace_bytes(rb, sb, T, inp.cfg.k, bm, lo, hi)
        assert need <= L.MOE_STATIC_SCRATCH_BYTES, (name, need)
        want = qm.moe_expert_forward(rb, sb, x, wd, al, lo, hi)
        out = torch.full((T, inp.cfg.H), float("nan"), dtype=torch.float32, device="cuda")
        got = qm.moe_expert_forward_static(rb, sb, x, wd, al, lo, hi, out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        # same kernels on the same inputs: identical bits, whatever the workspace held before
        assert torch.equal(got, want), name
        ref = O.expert_forward(inp.routed, inp.shared, inp.x, ids, w, lo, hi)
        check_close(f"static scratch {name}", got.cpu().numpy(), ref)


def test_static_scratch_rejects_calls_beyond_its_size():
    """A prefill batch whose workspace exceeds the fixed scratch fails with MOE_ERR_WORKSPACE
    before anything is enqueued; the same call with a caller workspace is accepted."""
    cfg = S.CONFIGS[3]
    T, bm = 8192, 128
    bank = qm.DeviceBank(cfg.fmt, cfg.E, cfg.H, cfg.I, *(torch.empty(16, dtype=torch.uint8, device="cuda")
                                                          for _ in range(4)),
                         torch.empty(16, device="cuda"), torch.empty(16, device="cuda"), qm.MOE_LAYOUT_TILE16)
    al = qm.alloc_align(T, cfg.k, cfg.E, bm)
    need = qm.moe_workspace_bytes(bank, None, T, cfg.k, bm, 0, cfg.I)
    assert need > L.MOE_STATIC_SCRATCH_BYTES
    x = torch.empty((T, cfg.H), dtype=torch.bfloat16, device="cuda")
    w = torch.empty((T, cfg.k), dtype=torch.float32, device="cuda")
    out = torch.empty((T, cfg.H), dtype=torch.float32, device="cuda")
    rs, als = bank.struct(), al.struct()
    rc = L.lib().moe_expert_forward_static(ctypes.byref(rs), None, ctypes.c_void_p(x.data_ptr()), T, cfg.k,
                                           ctypes.c_void_p(w.data_ptr()), ctypes.byref(als), 0, cfg.I,
                                           ctypes.c_void_p(out.data_ptr()), 0, None)
    assert rc == L.MOE_ERR_WORKSPACE
    assert b"scratch" in L.lib().moe_last_error()
