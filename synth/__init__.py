"""Seeded synthetic inputs shared by the oracle-side tests, the GPU path's tests and the bench.

This package holds no arithmetic of the ranker or the dynamic layer: it only draws random
embeddings, weights and tails, and converts fp32 values to bf16 bit patterns.
"""
from .inputs import (  # noqa: F401
    CONFIGS,
    Config,
    Inputs,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    layer_params,
    make_inputs,
    processor_params,
    n_splits,
)
