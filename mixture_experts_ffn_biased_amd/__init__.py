"""MI355X-native forward pass of one sparse mixture-of-experts feed-forward layer.

The layer runs as hand-written HIP kernels for gfx950 inside ``libmoe.so``
(C ABI in ``include/moe.h``); this package is its thin Python binding.
"""
from .binding import (MOE_N_STAGES, STAGES, MoeConfig, MoeError, alloc_workspace, lib,
                      alloc_block_workspace, moe_balance_update, moe_block_forward,
                      moe_block_forward_packed, moe_block_workspace_bytes, moe_check_cfg, moe_rmsnorm, moe_layer_forward, moe_layer_forward_ex,
                      moe_layer_forward_packed, moe_layer_forward_packed_ex, moe_pack_weights_ex,
                      moe_packed_weights_bytes_ex, moe_plan_describe_ex, moe_workspace_bytes_ex,
                      moe_pack_weights, moe_packed_weights_bytes, moe_plan_describe, moe_route_debug, moe_status_str,
                      moe_timing_enable, moe_timing_read, moe_workspace_bytes)

__all__ = ["MOE_N_STAGES", "STAGES", "MoeConfig", "MoeError", "alloc_workspace", "lib",
           "alloc_block_workspace", "moe_balance_update", "moe_block_forward", "moe_block_forward_packed",
           "moe_block_workspace_bytes", "moe_check_cfg", "moe_rmsnorm", "moe_layer_forward", "moe_layer_forward_ex",
           "moe_layer_forward_packed", "moe_layer_forward_packed_ex", "moe_pack_weights_ex",
           "moe_packed_weights_bytes_ex", "moe_plan_describe_ex", "moe_workspace_bytes_ex",
           "moe_pack_weights", "moe_packed_weights_bytes", "moe_plan_describe", "moe_route_debug", "moe_status_str",
           "moe_timing_enable", "moe_timing_read", "moe_workspace_bytes"]
