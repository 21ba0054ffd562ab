"""Seeded synthetic inputs for the routed-expert FFN (tests, smoke run, bench).

This package draws random numbers and stores them in the canonical (MLX-style)
layout. It holds none of the method's arithmetic: no dequantisation, no
routing, no expert math. Both the FP64 oracle and the HIP path are fed from it.
"""
from .gen import (  # noqa: F401
    QFormat, QTensor, Layer, ConfigSpec, CONFIGS, AFFINE, SYMMETRIC, DENSE,
    MXFP4, BF16, FP16, E8M0, MX4G32, make_layer, make_expert, make_x, make_tiny_config, words_per_row,
    f32_to_bf16_bits, f64_to_fp16_bits,
)
