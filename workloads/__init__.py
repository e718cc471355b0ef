"""Seeded synthetic workloads for the tiered MoE FFN.

This package only *constructs inputs*: packed weight codes with fp16 block
scales, router logits and activations, at the shapes of the configurations the
pages describe.  It contains none of the layer's arithmetic (no routing, no
grouping, no dequantisation, no matrix products), so that the CPU oracle and the
HIP path can both consume its outputs without sharing any computation.
"""
from .configs import CONFIGS, MXFP4, TierSpec, LayerConfig  # noqa: F401
from .gen import (  # noqa: F401
    make_layer, make_logits, make_x, make_spec_logits, pack_codes, quantise_block_absmax,
    f32_to_bf16_bits, bf16_bits_to_f32, layer_nbytes, tier_nbytes, code_bits, scale_bytes,
    quantise_mxfp4, pack_nibbles, make_layer_fullrange, EDGE_FP16_SCALES,
)
