"""Helpers of the GPU parity tests: upload synthetic inputs, run the HIP path through the
binding, and compare with the oracle at the stated tolerance."""
import numpy as np
import torch

import quantized_moe_expert_topk_amd as qm


def tol(ref: np.ndarray) -> float:
    """Output acceptance: max|delta| <= 1e-2 * max|ref| + 1e-3."""
    return 1e-2 * float(np.abs(ref).max()) + 1e-3


def to_dev(a: np.ndarray | None, dev="cuda"):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def device_bank(b, dev="cuda", packed=True) -> qm.DeviceBank:
    """Upload a row-major bank; by default reorder it into the kernels' tile-16 layout."""
    bank = qm.DeviceBank(b.fmt, b.E, b.H, b.I, to_dev(b.gate_up, dev), to_dev(b.gate_up_scale, dev),
                         to_dev(b.down, dev), to_dev(b.down_scale, dev), to_dev(b.gate_up_global, dev),
                         to_dev(b.down_global, dev))
    return qm.moe_pack_bank(bank) if packed else bank


def tile16_np(a: np.ndarray, unit: int) -> np.ndarray:
    """The MOE_LAYOUT_TILE16 order of a row-major [rows, pitch] byte matrix, written as an
    index transform: 16-row tiles, each stored as its units (of `unit` bytes) column by column."""
    R, P = a.shape
    return a.reshape(R // 16, 16, P // unit, unit).transpose(0, 2, 1, 3).reshape(R, P)


def bf16_dev(bits: np.ndarray, dev="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).to(dev)


def check_close(name, got: np.ndarray, ref: np.ndarray, report=None):
    assert got.shape == ref.shape, f"{name}: shape {got.shape} != {ref.shape}"
    if ref.size == 0:  # no tokens: nothing to compare beyond the shape
        print(f"[parity] {name}: empty {ref.shape}", flush=True)
        return 0.0
    err = float(np.abs(got.astype(np.float64) - ref).max())
    t = tol(ref)
    print(f"[parity] {name}: max|d|={err:.3e} tol={t:.3e} max|ref|={np.abs(ref).max():.3e} ratio={err / t:.3f}",
          flush=True)
    if report is not None:
        report[name] = dict(err=err, tol=t)
    assert err <= t, f"{name}: max|delta| {err:.3e} > tol {t:.3e}"
    return err


def align_np(al: qm.AlignOut) -> dict:
    return dict(sorted_ids=al.sorted_ids.cpu().numpy(), block_expert=al.block_expert.cpu().numpy(),
                counts=al.counts.cpu().numpy(), offsets=al.offsets.cpu().numpy(),
                total_padded=al.total_padded.cpu().numpy())
