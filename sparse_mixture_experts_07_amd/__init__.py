"""MI355X-native (gfx950) sparsely-gated MoE layer forward.

The layer y = sum_i G(x)_i E_i(x), G = softmax(KeepTopK(x W_g, k)), runs as
hand-written HIP kernels behind the C ABI in include/moe.h (libmoe.so in this
directory).  ``binding`` holds the ctypes entry points (same names as the C
calls); ``device`` holds torch-based device-memory plumbing.
"""
from . import binding
from .binding import (MoeConfig, MoeError, MoeWeights, config, config_of,
                      moe_abi_version, moe_combine, moe_expert_down,
                      moe_expert_ffn, moe_expert_up, moe_forward,
                      moe_grouped_rows, moe_load_stats, moe_param_counts,
                      moe_permute, moe_route, moe_status_string,
                      moe_workspace_bytes, weights)

__all__ = [
    "binding", "MoeConfig", "MoeError", "MoeWeights", "config", "config_of",
    "moe_abi_version", "moe_combine", "moe_expert_down", "moe_expert_ffn",
    "moe_expert_up", "moe_forward", "moe_grouped_rows", "moe_load_stats",
    "moe_param_counts", "moe_permute", "moe_route", "moe_status_string",
    "moe_workspace_bytes", "weights",
]
