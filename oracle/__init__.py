"""CPU oracle of the Mixtral sparse-MoE feed-forward layer.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check and
by the bench's CPU-baseline leg, never by the library.  See moe_oracle.py.
"""
from .moe_oracle import (  # noqa: F401
    router_logits, topk_indices, topk_mask, softmax, gating, silu, swiglu_expert,
    moe_layer, rmsnorm, round_bf16, moe_block, max_permuted_rows, group_by_expert,
    expert_rows, combine, routing_margin, top_gap, slot_order_gap,
)
from .fp8 import (  # noqa: F401
    e4m3_decode, e4m3_encode_rne, quantize_rows_fp8, dequantize_rows_fp8, moe_layer_fp8,
)
from .backward import backward_expert_rows, backward_token_rows, forward64, moe_layer_backward  # noqa: F401
