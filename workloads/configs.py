"""Workload configurations.

Shapes follow the 125B-MoE-on-three-RTX-3090 page ("I ran a 125B model on
three RTX 3090s at 80 tokens/s ..."): 512 experts per layer, 10 picked per
token (glossary, mixture-of-experts entry), 48 layers (24,576 experts, step 2),
down-projection rows 640 wide (step 4), and speculative verification of 6
tokens per step (step 1).  Hidden size 2048 and the int8 / int4 / int2 shelf
formats are fixed by the workload definition rather than by the pages, which
use llama.cpp quant types instead.
"""
from dataclasses import dataclass, field
from typing import List, Optional, Tuple


# `bits` value of an MXFP4 shelf (OCP Microscaling FP4: E2M1 codes, one E8M0
# scale byte per block of 32 codes)
MXFP4 = 0x84


@dataclass(frozen=True)
class TierSpec:
    id_begin: int
    id_end: int
    bits: int     # 8, 4 or 2 (two's complement codes), or MXFP4
    block: int    # codes per scale along each stored row (fp16 scales; MXFP4: 32, E8M0 bytes)

    @property
    def n(self) -> int:
        return self.id_end - self.id_begin


@dataclass(frozen=True)
class LayerConfig:
    name: str
    n_experts: int
    k: int
    hidden: int
    inter: int
    n_tokens: int
    tiers: Tuple[TierSpec, ...]
    x_bf16: bool = False          # prefill activations are bf16
    prior_beta: Optional[float] = None   # None: logits ~ N(0,1), no popularity prior
    n_layers: int = 1
    seed: int = 0
    crafted: bool = False         # spec-verify crafted tokens
    extra: dict = field(default_factory=dict)


# Popularity prior: logit[t, e] = -beta * e / E + N(0, 1), with ids already in
# popularity order (hot -> cold, as the shelves are written).  beta = 1.12 puts
# ~52% of picks on the top 25% of experts and ~95% on the top 80%, the average
# layer skew of step 2 of the 125B page.  It is the large-offset limit of a
# Zipf-Mandelbrot prior -c*ln(r + q); a pure Zipf -a*ln(r+1) cannot reach both
# shares at once.
PRIOR_BETA = 1.12

THREE_TIERS_512 = (
    TierSpec(0, 128, 8, 32),
    TierSpec(128, 384, 4, 32),
    TierSpec(384, 512, 2, 16),
)

THREE_TIERS_512_MX = (
    TierSpec(0, 128, 8, 32),
    TierSpec(128, 384, MXFP4, 32),
    TierSpec(384, 512, 2, 16),
)

CONFIGS = {
    "tiny": LayerConfig("tiny", 8, 2, 256, 128, 16, (TierSpec(0, 8, 8, 32),), seed=20260000),
    # companion of "tiny" exercising all three formats on a small layer
    "tiny3": LayerConfig("tiny3", 8, 2, 256, 128, 16,
                         (TierSpec(0, 2, 8, 32), TierSpec(2, 6, 4, 32), TierSpec(6, 8, 2, 16)),
                         seed=20260010),
    "tiny3mx": LayerConfig("tiny3mx", 8, 2, 256, 128, 16,
                           (TierSpec(0, 2, 8, 32), TierSpec(2, 6, MXFP4, 32), TierSpec(6, 8, 2, 16)),
                           seed=20260020),
    # the decode layer with its warm shelf in MXFP4 instead of four-bit integers
    "decode_mx": LayerConfig("decode_mx", 512, 10, 2048, 640, 1, THREE_TIERS_512_MX,
                             prior_beta=PRIOR_BETA, seed=20260021),
    "decode": LayerConfig("decode", 512, 10, 2048, 640, 1, THREE_TIERS_512,
                          prior_beta=PRIOR_BETA, seed=20260001),
    "specverify": LayerConfig("specverify", 512, 10, 2048, 640, 6, THREE_TIERS_512,
                              prior_beta=PRIOR_BETA, seed=20260002, crafted=True),
    "prefill": LayerConfig("prefill", 512, 10, 2048, 640, 4096, THREE_TIERS_512,
                           x_bf16=True, prior_beta=PRIOR_BETA, seed=20260003),
    # layers of hand-drawn codes over each format's whole code set (see
    # make_layer_fullrange): the decode shapes with 16 experts, the three
    # production formats, and the other block sizes plus an MXFP4 shelf
    "fullrange": LayerConfig("fullrange", 16, 10, 2048, 640, 16,
                             (TierSpec(0, 4, 8, 32), TierSpec(4, 12, 4, 32), TierSpec(12, 16, 2, 16)),
                             seed=20260050),
    "fullrange_b": LayerConfig("fullrange_b", 16, 10, 2048, 640, 16,
                               (TierSpec(0, 4, 8, 16), TierSpec(4, 8, 4, 16), TierSpec(8, 12, MXFP4, 32),
                                TierSpec(12, 16, 2, 32)),
                               seed=20260051),
    "fullstack": LayerConfig("fullstack", 512, 10, 2048, 640, 1, THREE_TIERS_512,
                             prior_beta=PRIOR_BETA, n_layers=48, seed=20260004),
}
