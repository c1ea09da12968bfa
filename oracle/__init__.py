"""CPU oracle of the routed-expert MoE layer.  TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The GPU library never imports it and shares no code with it.
"""
from .moe_oracle import (  # noqa: F401
    bf16_to_f32, unpack_codes, pack_codes, dequantize, router_logits, topk_softmax,
    permute, silu, expert_ffn, combine, moe_layer, moe_layer_tokens, rel_fro, unpack_fp6_fields, e2m3_value, FP6,
    e2m1_value, e4m3_value, round_e4m3, round_e2m1, quant_nvfp4, unpack_e2m1_fields, dequantize_nvfp4,
    expert_ffn_nvfp4, moe_layer_nvfp4, NVFP4_GROUP,
)
