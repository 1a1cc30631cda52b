"""Seeded synthetic workloads for the five decode projections.

This package only draws random inputs and states the workload sizes. It holds
none of the projection arithmetic, so both the CPU oracle and the GPU library
can be fed from it without sharing any code with each other.
"""

from .shapes import LAYERS, LAYER_ID, SHAPES, ROUTER, LOADS, AWKWARD_M, weight_dtype, out_dtype
from .generate import (
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    make_weight,
    make_x,
    XSample,
)

__all__ = [
    "LAYERS", "LAYER_ID", "SHAPES", "ROUTER", "LOADS", "AWKWARD_M",
    "weight_dtype", "out_dtype",
    "bf16_bits_from_f32", "f32_from_bf16_bits", "make_weight", "make_x", "XSample",
]
