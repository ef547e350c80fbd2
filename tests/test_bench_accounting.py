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
