"""Seeded synthetic workloads shared by the oracle-side tests and the GPU path.

This package holds shapes, seeds and random draws only: no attention
arithmetic.  Both the CPU oracle and the HIP path consume the arrays it
produces, so the two sides see bit-identical inputs.
"""
from .configs import CONFIGS, Config, get_config
from .gen import (
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    generate,
    round_to_dtype,
    tree_layout,
)

__all__ = [
    "CONFIGS",
    "Config",
    "get_config",
    "bf16_bits_to_f32",
    "f32_to_bf16_bits",
    "generate",
    "round_to_dtype",
    "tree_layout",
]
