"""CPU oracle of the routed-expert MoE layer.  TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library never imports it and shares no code with it.
"""
from .moe_oracle import (  # noqa: F401
    bf16_to_f32, unpack_codes, pack_codes, dequantize, router_logits, topk_softmax,
    permute, silu, expert_ffn, combine, moe_layer, moe_layer_tokens, rel_fro, unpack_fp6_fields, e2m3_value, FP6,
)
