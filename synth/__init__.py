"""Seeded synthetic inputs for the MoE decode/verify round.

This package only draws random numbers and lays them out in the library's
weight formats (4-bit codes in blocks of 32 with an fp16 scale and an fp16
minimum per block, or in 256-weight super-blocks with 6-bit sub-block scales
and minima).  It holds none of the round's arithmetic: no
dequantisation, no router, no top-k, no SwiGLU, no combine.  Both the CPU
oracle and the HIP path consume what it produces.
"""
from .inputs import (  # noqa: F401
    CONFIGS,
    ShapeConfig,
    LayerInputs,
    config,
    quantize_q4b32,
    quantize_q4s256,
    make_layer,
    make_activations,
    make_residency,
    derive_seed,
)
