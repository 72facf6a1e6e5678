"""MI355X (gfx950) sparse MoE-layer forward: hand-written HIP kernels behind a
C ABI (include/moe.h, libmoe.so) and a thin ctypes binding."""
from .binding import (moe_backward_workspace_size, moe_layer_backward, moe_layer_forward_train, moe_saved_bytes,
                      EXPORTED, MoEError, load, moe_balanced_ids, moe_block_forward, moe_combine, moe_expert_down, moe_expert_up,
                      moe_grouped_swiglu, moe_hidden_bytes, moe_layer_forward, moe_layer_forward_noalloc, moe_layer_forward_routed,
                      moe_permute, moe_rmsnorm, moe_rmsnorm_route, moe_route, moe_route_replay, moe_shared_ffn, moe_workspace_size, make_config,
                      status_string, workspace)

__all__ = ["moe_backward_workspace_size", "moe_layer_backward", "moe_layer_forward_train", "moe_saved_bytes",
           "EXPORTED", "MoEError", "load", "moe_balanced_ids", "moe_block_forward", "moe_combine", "moe_expert_down", "moe_expert_up",
           "moe_grouped_swiglu", "moe_hidden_bytes", "moe_layer_forward", "moe_layer_forward_noalloc", "moe_layer_forward_routed",
           "moe_permute", "moe_rmsnorm", "moe_rmsnorm_route", "moe_route", "moe_route_replay", "moe_shared_ffn", "moe_workspace_size", "make_config",
           "status_string", "workspace"]
