"""The five MoE-layer workloads, as plain parameter records.

Each record holds the layer's parameters in the notation of the kwkr.cn page on sparse
activation (news/623730, section 2: T tokens, d model dim, E experts, top-k, capacity factor c)
plus the expert hidden width d_ffn (section 3.1's ``hidden_dim``), the softmax
temperature tau of the Gumbel-softmax router ("Mixture of Experts (MoE) 原理与工程落地全指南",
lpnh.cn, section 2.2) and the storage dtype. Nothing here computes any part of
the method: the capacity, routing and statistics are left to the code under test.
"""
from __future__ import annotations

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class MoEShape:
    name: str
    T: int                  # tokens in the batch (the [B, S, d] input flattened to [T, d])
    d: int                  # model dimension
    E: int                  # number of experts
    k: int                  # experts chosen per token
    d_ffn: int              # expert hidden dimension (Linear d -> d_ffn -> d)
    capacity_factor: float  # c in C = ceil(c * k * T / E)
    temperature: float = 1.0
    gumbel: bool = False
    dtype: str = "bf16"     # storage of x, W_g, W1, W2 and y: "bf16" or "f32"
    seed: int = 0
    recipe: str = "gauss"   # input recipe: "gauss", "zipf_bias", "clusters"
    wg_std: float | None = 0.02   # router weight std; None means 1/sqrt(fan_in)

    def with_(self, **kw) -> "MoEShape":
        return replace(self, **kw)


CONFIGS: dict[str, MoEShape] = {
    # Tiny fp32 layer: correctness of routing, drops, outputs and the balance statistic.
    "tiny_fp32": MoEShape("tiny_fp32", T=256, d=128, E=4, k=2, d_ffn=512,
                          capacity_factor=1.25, dtype="f32"),
    # Mixtral-like 8-expert top-2 layer: near-balanced routing, compute-bound grouped GEMM.
    "mixtral_like": MoEShape("mixtral_like", T=4096, d=4096, E=8, k=2, d_ffn=14336,
                             capacity_factor=1.25),
    # Switch-style top-1 with a Zipf(1.1) per-expert logit bias: many experts overflow.
    "switch_skew": MoEShape("switch_skew", T=16384, d=1024, E=64, k=1, d_ffn=4096,
                            capacity_factor=1.0, recipe="zipf_bias", wg_std=None),
    # Decode-sized batch over many small experts: weight streaming, HBM-bound.
    "decode": MoEShape("decode", T=128, d=4096, E=64, k=2, d_ffn=1408,
                       capacity_factor=2.0, wg_std=None),
    # Gumbel-noised routing at temperature 0.5 over long-tail clustered token features.
    "gumbel_longtail": MoEShape("gumbel_longtail", T=65536, d=2048, E=16, k=2, d_ffn=8192,
                                capacity_factor=1.5, temperature=0.5, gumbel=True,
                                recipe="clusters"),
}

# The configuration the throughput figure is quoted on.
HEADLINE = "mixtral_like"
