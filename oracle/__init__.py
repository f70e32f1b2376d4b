"""CPU oracle of the MoE FFN layer forward pass (test infrastructure only).

Only the test-suite, the package smoke check and the benchmark's
``cpu_baseline`` leg may import this package.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (TOPK_THEN_SOFTMAX, SOFTMAX_THEN_TOPK, NEAR_TIE_GAP,
                         router_logits, select_topk, gate_weights, route,
                         capacity, assign, gather_rows, silu, expert_ffn,
                         grouped_ffn, combine, moe_forward,
                         moe_forward_tokens)
