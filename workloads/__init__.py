"""Seeded synthetic inputs for multi-adapter LoRA batches.

This package only draws random inputs (activations, adapter weights, adapter
ids, segment lengths, upstream gradients) and stores them as bf16 bit
patterns. It holds none of the LoRA arithmetic: the CPU oracle and the HIP
library both consume what it produces, and neither imports the other.
"""
from .gen import (  # noqa: F401
    Meta,
    Problem,
    CONFIG_NAMES,
    DECODE_PROJECTIONS,
    bf16_bits_from_f32,
    make_config,
    make_custom,
    make_c2_projections,
    make_meta,
)
