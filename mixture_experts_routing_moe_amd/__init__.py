"""libmoe: the Mixture-of-Experts layer forward (and its backward) on AMD MI355X (gfx950).

The compute lives in libmoe.so (hand-written HIP kernels behind the C ABI of
include/moe.h); this package only binds it to torch tensors.
"""

from ._lib import MOE_BF16, MOE_F32, MoeError, lib  # noqa: F401
from .moe import (  # noqa: F401
    moe_align,
    moe_align_inverse,
    moe_align_workspace_size,
    moe_combine,
    moe_ffn_down_combine,
    moe_ffn_down_combine_fused,
    moe_expert_ffn,
    moe_expert_ffn_backward,
    moe_expert_ffn_backward_workspace_size,
    moe_expert_ffn_workspace_size,
    moe_ffn_down,
    moe_ffn_down_splits,
    moe_ffn_gate_up,
    moe_indices_to_multihot,
    moe_indices_to_multihot_backward,
    moe_layer,
    moe_layer_backward,
    moe_multihot_to_indices,
    moe_route,
    moe_route_align,
    moe_route_align_fused,
    moe_route_align_inverse,
    moe_route_align_gate_up,
    moe_route_align_gate_up_fused,
    moe_route_align_noalloc,
    moe_tile_schedule,
    moe_tile_schedule_max,
    moe_route_backward,
    moe_route_grouped_backward,
    moe_route_grouped,
    moe_route_multihot,
    moe_route_multihot_fused,
    moe_router_backward,
    moe_router_route,
)
