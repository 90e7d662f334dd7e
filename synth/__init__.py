"""Seeded synthetic inputs for the MoE-LoRA expert layer.

This package is shared by the CPU oracle and the HIP path.  It holds only
shapes, random draws and the fp32 -> bf16 / fp16 storage encodings of those draws;
none of the layer's arithmetic lives here.
"""
from .configs import (  # noqa: F401
    CONFIGS,
    LayerDims,
    LayerInputs,
    bf16_bits_from_f32,
    f16_bits_from_f32,
    make_inputs,
    make_logits,
)
