"""The synthetic workloads: one routed MoE layer at several shapes.

Distributions (the input recipe):
  * hidden states: fp32 N(0, 1) per element, then each token row RMS-normalised;
  * router gate [E, d]: N(0, 1/sqrt(d)) (standard deviation), stored fp32 for
    the tiny layer and bf16 for the others;
  * expert gate/up [E, f, d] and down [E, d, f]: fp32 N(0, 0.02), quantised
    to 4-bit affine codes, group 64 along the input axis, bf16 scale/bias;
  * top-k weights renormalised to sum 1 (norm_topk_prob) throughout.
"""
from __future__ import annotations

import dataclasses
import math


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    d_model: int
    num_experts: int
    top_k: int
    ffn_dim: int
    batch: int
    router_bf16: bool
    fused: bool = False
    norm_topk_prob: bool = True
    expert_sigma: float = 0.02
    seed: int = 0
    num_layers: int = 1
    shared_ffn_dim: int = 0       # 0: no shared expert

    @property
    def router_sigma(self) -> float:
        return 1.0 / math.sqrt(self.d_model)

    @property
    def pairs(self) -> int:
        return self.batch * self.top_k

    def expert_bytes(self) -> int:
        """Packed words + bf16 scales + bf16 biases of one expert (gate, up, down)."""
        d, f = self.d_model, self.ffn_dim
        return 3 * (f * d // 2 + 2 * 2 * f * d // 64)

    def expert_packed_bytes(self) -> int:
        return 3 * self.ffn_dim * self.d_model // 2

    def with_batch(self, batch: int) -> "LayerConfig":
        return dataclasses.replace(self, batch=batch)


# d=256, 16 experts, top-4, ffn 128, 8 tokens, fp32 router.
TINY = LayerConfig("tiny_d256_e16_k4_f128", 256, 16, 4, 128, 8, router_bf16=False)
# Qwen3-235B-shaped layer: d=4096, 128 experts, top-8, ffn 1536; decode and prefill chunk.
DECODE = LayerConfig("d4096_e128_k8_f1536_b1", 4096, 128, 8, 1536, 1, router_bf16=True)
PREFILL = dataclasses.replace(DECODE, name="d4096_e128_k8_f1536_b64", batch=64)
# 256-expert layer with the fused gate_up layout.
FUSED_B1 = LayerConfig("fused_d2048_e256_k8_f512_b1", 2048, 256, 8, 512, 1, router_bf16=True,
                       fused=True)
FUSED_B64 = dataclasses.replace(FUSED_B1, name="fused_d2048_e256_k8_f512_b64", batch=64)
# Stacked routed-expert path: 94 layers of the decode shape.
STACK = dataclasses.replace(DECODE, name="stack94_d4096_e128_k8_f1536", num_layers=94)

# The decode layer with a shared expert twice the routed width (an always-active
# expert beside the routed ones, as in architectures that have one).
DECODE_SHARED = dataclasses.replace(DECODE, name="d4096_e128_k8_f1536_s3072_b1",
                                    shared_ffn_dim=3072)
PREFILL_SHARED = dataclasses.replace(DECODE_SHARED, name="d4096_e128_k8_f1536_s3072_b64",
                                     batch=64)

ALL = {c.name: c for c in (TINY, DECODE, PREFILL, FUSED_B1, FUSED_B64, STACK, DECODE_SHARED,
                           PREFILL_SHARED)}


def expected_union(E: int, K: int, B: int) -> float:
    """E[|U|] for B tokens each routed to K distinct experts, uniformly: each
    expert is missed by a token with probability 1 - K/E."""
    return E * (1.0 - (1.0 - K / E) ** B)
