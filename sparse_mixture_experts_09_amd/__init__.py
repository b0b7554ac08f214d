"""Token-choice Mixture-of-Experts FFN layer forward on MI355X (gfx950).

The layer runs in libmoe.so (hand-written HIP); this package is its build
script and ctypes binding. See include/moe.h for the C interface.
"""
from .moe import (MoeError, lib, moe_capacity, moe_expert_down, moe_expert_gate_up, moe_ffn_workspace_bytes, moe_forward, moe_grouped_ffn, moe_permute,  # noqa: F401
                  moe_permute_priority_workspace_bytes, moe_permute_workspace_bytes, moe_route, moe_rows_max, moe_unpermute_combine,
                  moe_workspace_bytes, status_string, moe_route_expert_choice, moe_gather_rows,
                  moe_grouped_ffn_rows, moe_combine_expert_choice, moe_forward_expert_choice, moe_backward,
                  moe_permute_noalloc, moe_permute_noalloc_scratch_bytes, moe_backward_expert_choice)
