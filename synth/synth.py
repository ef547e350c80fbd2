"""Seeded synthetic inputs for the quantized MoE expert layer (input side only).

Everything here produces the bytes that both the CPU oracle and the GPU library consume:
bf16 activations, bf16 router weights, an optional fp32 router bias, and quantized expert
banks in the layouts the FreeToken pages describe (gate_up ``[2I, H]`` with gate rows
``[0, I)`` and up rows ``[I, 2I)``, down ``[H, I]``; issue #520 section 4 "Expert sharding"
and the nvfp4.py hunk of its patch; issue #62 "What it touches" item 1).  None of the
layer's arithmetic lives here; the generators and quantizers are in ``synth.c``.

The layer configurations below are the synthetic workloads: shapes follow the models the
pages run (Qwen3.6-35B-A3B: hidden 2048, 256 experts, top-8, expert and shared intermediate
512, issue #520 section 2; DeepSeek-V4-Flash routed FP4 experts with 32-element scale
blocks, PR #70 "Checkpoint loading"), with N(0, 0.02) weights and N(0, 1) tokens.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")

# stream tags: (seed, tag, index) keys one counter-based stream
TAG_X, TAG_ROUTER, TAG_ZIPF, TAG_GATE_UP, TAG_DOWN = 1, 2, 3, 4, 5
TAG_SH_GATE_UP, TAG_SH_DOWN, TAG_LOGITS, TAG_IDS = 6, 7, 8, 9

WEIGHT_SIGMA = 0.02


def build(force: bool = False) -> str:
    """Compile ``libsynth.so`` next to this file (plain C, gcc, OpenMP)."""
    src = os.path.join(_HERE, "synth.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        cmd = f"gcc -O2 -fopenmp -fPIC -shared -o {_LIB_PATH}.tmp {src} -lm && mv {_LIB_PATH}.tmp {_LIB_PATH}"
        if os.system(cmd) != 0:
            raise RuntimeError(f"synth build failed: {cmd}")
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        u64, u32, i32, i64, dbl = (ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int32,
                                   ctypes.c_int64, ctypes.c_double)
        vp = ctypes.c_void_p
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64, u32, u32]
        L.synth_normal_f64.argtypes = [u64, u32, u32, i64, i64, dbl, vp]
        L.synth_uniform_f64.argtypes = [u64, u32, u32, i64, i64, vp]
        L.synth_bf16_normal.argtypes = [u64, u32, u32, dbl, i64, vp]
        L.synth_nvfp4_matrix.argtypes = [u64, u32, u32, i32, i32, dbl, vp, vp, vp]
        L.synth_fp8blk_matrix.argtypes = [u64, u32, u32, i32, i32, dbl, vp, vp]
        L.synth_mxfp4_matrix.argtypes = [u64, u32, u32, i32, i32, dbl, vp, vp]
        L.synth_q4_0_matrix.argtypes = [u64, u32, u32, i32, i32, dbl, vp, vp]
        L.synth_zipf_bias.argtypes = [u64, u32, i32, dbl, vp]
        L.synth_randint.argtypes = [u64, u32, u32, i64, i32, vp]
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


# ----------------------------------------------------------------------------- tensors

def normal_f64(seed: int, tag: int, index: int, n: int, sigma: float = 1.0, start: int = 0) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().synth_normal_f64(seed, tag, index, start, n, sigma, _p(out))
    return out


def uniform_f64(seed: int, tag: int, index: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, np.float64)
    lib().synth_uniform_f64(seed, tag, index, start, n, _p(out))
    return out


def bf16_normal(seed: int, tag: int, index: int, shape, sigma: float) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(0, sigma^2) numbers."""
    out = np.empty(shape, np.uint16)
    lib().synth_bf16_normal(seed, tag, index, sigma, out.size, _p(out))
    return out


def tokens(seed: int, T: int, H: int, batch: int = 0) -> np.ndarray:
    """Token batch ``batch``: bf16 [T, H] from N(0, 1)."""
    return bf16_normal(seed, TAG_X, batch, (T, H), 1.0)


def router_weight(seed: int, E: int, H: int) -> np.ndarray:
    """Router weight: bf16 [E, H] from N(0, 0.02^2)."""
    return bf16_normal(seed, TAG_ROUTER, 0, (E, H), WEIGHT_SIGMA)


def zipf_bias(seed: int, E: int, s: float) -> np.ndarray:
    out = np.empty(E, np.float32)
    lib().synth_zipf_bias(seed, TAG_ZIPF, E, s, _p(out))
    return out


def randint(seed: int, index: int, count: int, n: int) -> np.ndarray:
    out = np.empty(count, np.int32)
    lib().synth_randint(seed, TAG_IDS, index, count, n, _p(out))
    return out


def logits_f32(seed: int, index: int, T: int, E: int) -> np.ndarray:
    """Standalone fp32 logits (N(0,1)) for tests of selection from given logits."""
    return normal_f64(seed, TAG_LOGITS, index, T * E).astype(np.float32).reshape(T, E)


# ----------------------------------------------------------------------------- banks

FORMATS = ("nvfp4", "fp8blk", "mxfp4", "bf16", "q4_0")


@dataclass
class Bank:
    """E experts in the full-I layout.  Arrays are numpy, C-contiguous, expert-major."""
    fmt: str
    E: int
    H: int
    I: int
    gate_up: np.ndarray            # nvfp4/mxfp4: u8 [E, 2I, H/2]; fp8blk: u8 [E, 2I, H]; bf16: u16 bits [E, 2I, H]
    gate_up_scale: np.ndarray      # nvfp4: u8 e4m3 [E, 2I, H/16]; fp8blk: f32 [E, 2I/128, H/128]; mxfp4: u8 e8m0 [E, 2I, H/32]
    down: np.ndarray               # nvfp4/mxfp4: u8 [E, H, I/2]; fp8blk: u8 [E, H, I]
    down_scale: np.ndarray         # nvfp4: u8 [E, H, I/16]; fp8blk: f32 [E, H/128, I/128]; mxfp4: u8 [E, H, I/32]
    gate_up_global: np.ndarray | None = None   # nvfp4 only: f32 [E, 2I]
    down_global: np.ndarray | None = None      # nvfp4 only: f32 [E, H]

    def arrays(self):
        return {k: getattr(self, k) for k in ("gate_up", "gate_up_scale", "gate_up_global",
                                              "down", "down_scale", "down_global")}

    def nbytes_expert(self) -> int:
        return sum(a[0].nbytes for a in self.arrays().values() if a is not None)


def _alloc_bank(fmt: str, E: int, H: int, I: int) -> Bank:
    if fmt == "nvfp4":
        return Bank(fmt, E, H, I,
                    gate_up=np.zeros((E, 2 * I, H // 2), np.uint8),
                    gate_up_scale=np.zeros((E, 2 * I, H // 16), np.uint8),
                    down=np.zeros((E, H, I // 2), np.uint8),
                    down_scale=np.zeros((E, H, I // 16), np.uint8),
                    gate_up_global=np.zeros((E, 2 * I), np.float32),
                    down_global=np.zeros((E, H), np.float32))
    if fmt == "fp8blk":
        return Bank(fmt, E, H, I,
                    gate_up=np.zeros((E, 2 * I, H), np.uint8),
                    gate_up_scale=np.zeros((E, 2 * I // 128, H // 128), np.float32),
                    down=np.zeros((E, H, I), np.uint8),
                    down_scale=np.zeros((E, H // 128, I // 128), np.float32))
    if fmt == "mxfp4":
        return Bank(fmt, E, H, I,
                    gate_up=np.zeros((E, 2 * I, H // 2), np.uint8),
                    gate_up_scale=np.zeros((E, 2 * I, H // 32), np.uint8),
                    down=np.zeros((E, H, I // 2), np.uint8),
                    down_scale=np.zeros((E, H, I // 32), np.uint8))
    if fmt == "q4_0":  # codes as FP4 (llama.cpp block order), fp16 d bits per 32
        return Bank(fmt, E, H, I,
                    gate_up=np.zeros((E, 2 * I, H // 2), np.uint8),
                    gate_up_scale=np.zeros((E, 2 * I, H // 32), np.uint16),
                    down=np.zeros((E, H, I // 2), np.uint8),
                    down_scale=np.zeros((E, H, I // 32), np.uint16))
    if fmt == "bf16":  # unquantized: no scales (empty placeholders keep the arrays uniform)
        return Bank(fmt, E, H, I,
                    gate_up=np.zeros((E, 2 * I, H), np.uint16),
                    gate_up_scale=np.zeros((E, 0), np.uint8),
                    down=np.zeros((E, H, I), np.uint16),
                    down_scale=np.zeros((E, 0), np.uint8))
    raise ValueError(f"unknown format {fmt!r}")


def _fill_expert(b: Bank, e: int, seed: int, tag_gu: int, tag_dn: int, index: int) -> None:
    L = lib()
    H, I, s = b.H, b.I, WEIGHT_SIGMA
    if b.fmt == "nvfp4":
        L.synth_nvfp4_matrix(seed, tag_gu, index, 2 * I, H, s, _p(b.gate_up[e]), _p(b.gate_up_scale[e]),
                             _p(b.gate_up_global[e]))
        L.synth_nvfp4_matrix(seed, tag_dn, index, H, I, s, _p(b.down[e]), _p(b.down_scale[e]),
                             _p(b.down_global[e]))
    elif b.fmt == "fp8blk":
        L.synth_fp8blk_matrix(seed, tag_gu, index, 2 * I, H, s, _p(b.gate_up[e]), _p(b.gate_up_scale[e]))
        L.synth_fp8blk_matrix(seed, tag_dn, index, H, I, s, _p(b.down[e]), _p(b.down_scale[e]))
    elif b.fmt == "q4_0":
        L.synth_q4_0_matrix(seed, tag_gu, index, 2 * I, H, s, _p(b.gate_up[e]), _p(b.gate_up_scale[e]))
        L.synth_q4_0_matrix(seed, tag_dn, index, H, I, s, _p(b.down[e]), _p(b.down_scale[e]))
    elif b.fmt == "bf16":
        b.gate_up[e] = bf16_normal(seed, tag_gu, index, (2 * I, H), s)
        b.down[e] = bf16_normal(seed, tag_dn, index, (H, I), s)
    else:
        L.synth_mxfp4_matrix(seed, tag_gu, index, 2 * I, H, s, _p(b.gate_up[e]), _p(b.gate_up_scale[e]))
        L.synth_mxfp4_matrix(seed, tag_dn, index, H, I, s, _p(b.down[e]), _p(b.down_scale[e]))


def routed_bank(seed: int, fmt: str, E: int, H: int, I: int, experts=None) -> Bank:
    """Routed bank; expert e's weights come from streams (seed, GATE_UP/DOWN, e).
    ``experts`` limits generation to a subset (the others stay zero)."""
    b = _alloc_bank(fmt, E, H, I)
    for e in (range(E) if experts is None else sorted(set(int(v) for v in experts))):
        _fill_expert(b, e, seed, TAG_GATE_UP, TAG_DOWN, e)
    return b


def shared_bank(seed: int, fmt: str, H: int, I: int) -> Bank:
    """The shared expert as a one-expert bank (streams SH_GATE_UP/SH_DOWN, index 0)."""
    b = _alloc_bank(fmt, 1, H, I)
    _fill_expert(b, 0, seed, TAG_SH_GATE_UP, TAG_SH_DOWN, 0)
    return b


def slice_bank(b: Bank, lo: int, hi: int) -> Bank:
    """A rank's own storage for the slice [lo, hi): gate rows [lo,hi) and up rows
    [I+lo, I+hi) with their scale rows / globals; down columns [lo, hi) with the matching
    scale columns; down_global replicated (PR #637 "Implementation notes": a companion is
    split along its weight's axis when it has that axis, replicated otherwise).
    Copies, never views (issue #520 section 4, ".clone()")."""
    I, Il = b.I, hi - lo
    gu_rows = np.r_[lo:hi, I + lo:I + hi]
    if b.fmt == "bf16":
        return Bank(b.fmt, b.E, b.H, Il,
                    gate_up=np.ascontiguousarray(b.gate_up[:, gu_rows]),
                    gate_up_scale=b.gate_up_scale.copy(),
                    down=np.ascontiguousarray(b.down[:, :, lo:hi]),
                    down_scale=b.down_scale.copy())
    if b.fmt == "fp8blk":
        blk_rows = np.r_[lo // 128:hi // 128, (I + lo) // 128:(I + hi) // 128]
        return Bank(b.fmt, b.E, b.H, Il,
                    gate_up=np.ascontiguousarray(b.gate_up[:, gu_rows]),
                    gate_up_scale=np.ascontiguousarray(b.gate_up_scale[:, blk_rows]),
                    down=np.ascontiguousarray(b.down[:, :, lo:hi]),
                    down_scale=np.ascontiguousarray(b.down_scale[:, :, lo // 128:hi // 128]))
    grp = 16 if b.fmt == "nvfp4" else 32
    out = Bank(b.fmt, b.E, b.H, Il,
               gate_up=np.ascontiguousarray(b.gate_up[:, gu_rows]),
               gate_up_scale=np.ascontiguousarray(b.gate_up_scale[:, gu_rows]),
               down=np.ascontiguousarray(b.down[:, :, lo // 2:hi // 2]),
               down_scale=np.ascontiguousarray(b.down_scale[:, :, lo // grp:hi // grp]))
    if b.fmt == "nvfp4":
        out.gate_up_global = np.ascontiguousarray(b.gate_up_global[:, gu_rows])
        out.down_global = b.down_global.copy()
    return out


# ----------------------------------------------------------------------------- configs

@dataclass(frozen=True)
class LayerConfig:
    cid: int
    name: str
    fmt: str
    H: int
    E: int
    k: int
    I: int
    shared: bool
    Ts: tuple
    slices: tuple            # (lo, hi) pairs; the first is the primary one
    zipf_s: float | None = None
    renormalize: bool = True

    @property
    def seed(self) -> int:
        return 1000 + self.cid


CONFIGS = {
    1: LayerConfig(1, "tiny NVFP4 layer H=256 E=8 top-2 I=128", "nvfp4", 256, 8, 2, 128, False,
                   (16,), ((0, 128), (0, 64), (64, 128))),
    2: LayerConfig(2, "Qwen3.6-35B-A3B-shaped NVFP4 decode layer H=2048 E=256 top-8 I=512 + shared I=512",
                   "nvfp4", 2048, 256, 8, 512, True, (1, 8, 32, 64), ((0, 256), (0, 512))),
    3: LayerConfig(3, "Qwen3.6-35B-A3B-shaped NVFP4 prefill layer T=8192, Zipf(1.1) router bias",
                   "nvfp4", 2048, 256, 8, 512, True, (8192,), ((0, 512), (0, 256)), zipf_s=1.1),
    4: LayerConfig(4, "fp8-block (128x128) expert layer H=2048 E=256 top-8 I=512", "fp8blk",
                   2048, 256, 8, 512, False, (1, 64, 4096), ((0, 256), (0, 512))),
    5: LayerConfig(5, "DeepSeek-V4-Flash-shaped MXFP4 (e8m0 per 32) layer H=4096 E=256 top-8 I=2048 + shared",
                   "mxfp4", 4096, 256, 8, 2048, True, (1, 16, 256), ((0, 1024), (0, 2048))),
    6: LayerConfig(6, "Qwen3.6-35B-A3B-shaped bf16 stacked-expert layer H=2048 E=256 top-8 I=512 + shared",
                   "bf16", 2048, 256, 8, 512, True, (1, 64, 8192), ((0, 256), (0, 512))),
    7: LayerConfig(7, "Qwen3.6-35B-A3B-shaped q4_0 (32-element blocks) expert layer H=2048 E=256 top-8 I=512",
                   "q4_0", 2048, 256, 8, 512, False, (1, 64), ((0, 256), (0, 512))),
}


@dataclass
class LayerInputs:
    cfg: LayerConfig
    x: np.ndarray                  # bf16 bits [T, H]
    router: np.ndarray             # bf16 bits [E, H]
    bias: np.ndarray | None        # f32 [E]
    routed: Bank
    shared: Bank | None = None
    extra: dict = field(default_factory=dict)


def layer_inputs(cfg: LayerConfig, T: int, batch: int = 0, experts=None, instance: int = 0) -> LayerInputs:
    """All inputs of one layer call.  ``instance`` selects an independently seeded layer
    (different weights) for cache-defeating rotation; ``experts`` restricts which routed
    experts are materialised (others are zero and must not be selected)."""
    seed = cfg.seed + 7919 * instance
    x = tokens(cfg.seed, T, cfg.H, batch)
    wr = router_weight(seed, cfg.E, cfg.H)
    bias = zipf_bias(seed, cfg.E, cfg.zipf_s) if cfg.zipf_s else None
    routed = routed_bank(seed, cfg.fmt, cfg.E, cfg.H, cfg.I, experts)
    shared = shared_bank(seed, cfg.fmt, cfg.H, cfg.I) if cfg.shared else None
    return LayerInputs(cfg, x, wr, bias, routed, shared)
