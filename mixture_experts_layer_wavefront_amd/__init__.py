"""MI355X (gfx950) forward and backward passes of one sparsely-gated MoE FFN
layer.

The layer runs in the HIP library libmoe_mi355x.so behind the C ABI of
include/moe.h; this package is its ctypes binding (``binding``), the build
script (``build``) and the seeded synthetic inputs (``workloads``).
"""
from .binding import (MOE_BF16, MOE_F32, MOE_SOFTMAX_THEN_TOPK,  # noqa: F401
                      MOE_TOPK_THEN_SOFTMAX, MoeError, Problem, capacity,
                      forward_shared_workspace_bytes,
                      grouped_ffn_workspace_bytes, load, moe_combine,
                      moe_forward, moe_forward_shared, moe_forward_stats,
                      moe_grouped_ffn, moe_grouped_ffn_rows, moe_grouped_ffn_scaled,
                      moe_forward_scaled,
                      moe_permute, moe_route, moe_route_stats,
                      forward_stats_workspace_bytes, route_stats_workspace_bytes,
                      permute_workspace_bytes, problem, route_workspace_bytes,
                      rows_bound, workspace_bytes,
                      train_state_bytes, backward_workspace_bytes,
                      moe_forward_train, moe_backward)
