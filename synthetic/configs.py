"""Workload shapes for the sparsely-gated MoE layer forward.

Five synthetic layers, from a tiny fp32 layer that a slow CPU loop finishes
in well under a second to layers with the shapes of GPT-2, Mixtral-8x7B, a
gpt-oss-20b decode step and DeepSeek-V3.  The shapes follow the models the
pages name (the Go book chapter "MoE", table of real MoE models; the
transformers-v5 article, sections on gpt-oss-20b and packed expert weights);
the value distributions are the synthetic recipe in ``synthetic.generate``.

This module holds sizes only: no arithmetic of the method.
"""
from dataclasses import dataclass, replace

GELU = 0
SWIGLU = 1
F32 = 0
BF16 = 1
# how the kept gate values are formed from the router scores
GATE_TOPK_SOFTMAX = 0    # softmax over the k kept scores (bias in both)
GATE_BIAS_SELECTS = 1    # bias steers the selection only; softmax of unbiased kept scores
GATE_SOFTMAX_ALL = 2     # softmax over all E scores, kept values not renormalised


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int            # tokens in the batch
    d: int            # d_model
    h: int            # d_hidden of one expert
    E: int            # routed experts
    k: int            # experts kept per token
    act: int          # GELU or SWIGLU
    dtype: int        # F32 or BF16 for x, expert weights, y
    S: int = 0        # shared always-on experts (0 or 1)
    router_bias: str = "none"   # "none" | "normal0.5" | "zipf1.1"
    layernorm_x: bool = False   # x drawn N(0,1) then LayerNorm'd per row
    expert_bias: bool = False   # GELU experts carry b1/b2 (zero-filled)
    seed: int = 0
    gate: int = GATE_TOPK_SOFTMAX

    @property
    def n_up(self) -> int:
        return self.h if self.act == GELU else 2 * self.h

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)

    def expert_flops(self) -> int:
        """Algorithmic FLOPs of the expert FFNs (routed + shared), no padding."""
        per_row = 2 * (self.d * self.n_up + self.h * self.d)
        return per_row * (self.T * self.k + self.S * self.T)


TINY = LayerConfig("tiny-fp32", T=64, d=64, h=256, E=8, k=2, act=GELU,
                   dtype=F32, expert_bias=True)
GPT2 = LayerConfig("gpt2-moe", T=6144, d=768, h=3072, E=6, k=2, act=GELU,
                   dtype=BF16, layernorm_x=True)
MIXTRAL = LayerConfig("mixtral-8x7b", T=4096, d=4096, h=14336, E=8, k=2,
                      act=SWIGLU, dtype=BF16, router_bias="normal0.5")
GPTOSS_DECODE = LayerConfig("gpt-oss-20b-decode", T=64, d=2880, h=2880, E=32,
                            k=4, act=SWIGLU, dtype=BF16)
DEEPSEEK_V3 = LayerConfig("deepseek-v3", T=8192, d=7168, h=2048, E=256, k=8,
                          act=SWIGLU, dtype=BF16, S=1, router_bias="zipf1.1")

ALL = [TINY, GPT2, MIXTRAL, GPTOSS_DECODE, DEEPSEEK_V3]
BY_NAME = {c.name: c for c in ALL}
