"""The bench's algorithmic byte counts (the roofline numerator) equal the bytes of the arrays a
rank actually holds for one expert's slice, for every format.  CPU only."""
import importlib.util
import os

import numpy as np
import pytest

from synth import synth as S

_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(_ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


def _nbytes(*arrays):
    return sum(a.nbytes for a in arrays if a is not None and a.size)


@pytest.mark.parametrize("fmt", ["nvfp4", "fp8blk", "mxfp4", "bf16", "q4_0"])
@pytest.mark.parametrize("H,I,lo,hi", [(256, 256, 0, 128), (512, 512, 128, 384), (384, 256, 0, 256)])
def test_expert_slice_bytes_match_a_rank_slice(fmt, H, I, lo, hi):
    b = S.slice_bank(S.routed_bank(5, fmt, 1, H, I), lo, hi)
    Il = hi - lo
    gate_up = _nbytes(b.gate_up, b.gate_up_global)
    down = _nbytes(b.down, b.down_global)
    if fmt != "fp8blk":  # per-row scales follow their rows
        gate_up += _nbytes(b.gate_up_scale)
        down += _nbytes(b.down_scale)
    else:  # one fp32 per 128 x 128 block: the count is the block area's share
        gate_up += 4 * (2 * Il * H) // 16384
        down += 4 * (H * Il) // 16384
    assert bench.gate_up_slice_bytes(fmt, H, Il) == gate_up
    assert bench.expert_slice_bytes(fmt, H, Il) == gate_up + down


def test_kernel_source_hash_ignores_comments_not_code(tmp_path, monkeypatch):
    """The traffic counters are keyed on the kernel's code and compiler options: an edit to
    comments or whitespace keeps the key, an edit to code or to a file's options changes it,
    and each kernel hashes its own sources."""
    from quantized_moe_expert_topk_amd import build as qbuild
    csrc = tmp_path / "quantized_moe_expert_topk_amd" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "device_common.h").write_text("#pragma once\nint helper(int x) { return x + 1; }\n")
    (csrc / "expert_kernels.h").write_text("// streaming\n__global__ void k(int *p) { p[0] = 1; }\n")
    (csrc / "expert_mxfp4.hip").write_text('#include "expert_kernels.h"\n')
    (csrc / "route_align_dev.h").write_text("#pragma once\nint rank(int x) { return x; }\n")
    (csrc / "expert_wide.hip").write_text("/* wide */\n__global__ void w(int *p) { p[0] = 2; }\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0, w0 = bench.kernel_source_hash("k_gate_up"), bench.kernel_source_hash("k_gate_up_wide")
    assert h0 != w0
    (csrc / "expert_kernels.h").write_text("// streaming kernels, reworded\n/* block\n comment */\n"
                                           "__global__ void k(int *p) {   p[0] = 1;   }  // trailing\n")
    assert bench.kernel_source_hash("k_gate_up") == h0
    (csrc / "expert_kernels.h").write_text("__global__ void k(int *p) { p[0] = 3; }\n")
    h1 = bench.kernel_source_hash("k_gate_up")
    assert h1 != h0
    assert bench.kernel_source_hash("k_gate_up_wide") == w0
    monkeypatch.setitem(qbuild.FILE_FLAGS, "expert_mxfp4.hip", ["-mllvm", "-some-other-option"])
    assert bench.kernel_source_hash("k_gate_up") != h1
    (csrc / "device_common.h").write_text("#pragma once\nint helper(int x) { return x + 2; }\n")
    assert bench.kernel_source_hash("k_gate_up_wide") != w0
    h2 = bench.kernel_source_hash("k_gate_up")
    (csrc / "route_align_dev.h").write_text("#pragma once\nint rank(int x) { return -x; }\n")
    assert bench.kernel_source_hash("k_gate_up") != h2  # the routing helpers gate_up includes
