"""CPU oracle of the MoE verify step: test infrastructure only.

Importable by the tests, by the package smoke check and by the benchmark's
CPU-baseline leg; never by the GPU library or its binding.
"""
from .moe_oracle import (  # noqa: F401
    as_fp32, forward_tokens, fp32_to_bf16_rne, gate_weights, lm_head_argmax,
    moe_layer, rms_norm, router_logits, select_top_k, silu, spec_accept, store,
    swiglu_expert, verify_step, widen,
)
