"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle."""
from .configs import (ALL, BY_NAME, BF16, DEEPSEEK_V3, F32, GATE_BIAS_SELECTS,
                      GATE_SOFTMAX_ALL, GATE_TOPK_SOFTMAX, GELU, GPT2,
                      GPTOSS_DECODE, MIXTRAL, SWIGLU, TINY, LayerConfig)
from .generate import (LayerInputs, bf16_bits_to_f32, f32_to_bf16_bits,
                       make_inputs, make_noisy_gate, zipf_log_bias)

__all__ = [
    "ALL", "BY_NAME", "BF16", "DEEPSEEK_V3", "F32", "GATE_BIAS_SELECTS",
    "GATE_SOFTMAX_ALL", "GATE_TOPK_SOFTMAX", "GELU", "GPT2",
    "GPTOSS_DECODE", "MIXTRAL", "SWIGLU", "TINY", "LayerConfig", "LayerInputs",
    "bf16_bits_to_f32", "f32_to_bf16_bits", "make_inputs", "make_noisy_gate", "zipf_log_bias",
]
