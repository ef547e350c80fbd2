"""MI355X (gfx950) quantized MoE expert layer on one rank's intermediate-dimension slice.

The compute lives in ``libqmoe.so`` (hand-written HIP kernels behind the C ABI of
``include/qmoe.h``); this package is its Python binding.
"""
from ._lib import (EXPORTS, LIB_PATH, MOE_LAYOUT_MXFP4_T, MOE_LAYOUT_ROWS, MOE_LAYOUT_TILE16,  # noqa: F401
                   MoeError, lib)
from .api import (AlignOut, DeviceBank, MoeLayer, alloc_align, choose_block_m, moe_align,  # noqa: F401
                  moe_align_capacity, moe_align_workspace_bytes, moe_expert_down, moe_expert_forward,
                  moe_expert_forward_static,
                  moe_expert_gate_up, moe_layer_forward, moe_pack_bank, moe_route, moe_route_align,
                  moe_route_align_workspace_bytes,
                  moe_route_from_logits, moe_route_workspace_bytes, moe_workspace_bytes)
