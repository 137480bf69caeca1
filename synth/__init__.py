"""Seeded synthetic inputs shared by the CPU oracle side and the HIP side.

This package only draws random numbers and lays them out: activations, fp32
weights, raw packed words and the layer shapes. It holds none of the quantised
linear layer's arithmetic (no scales, no codes, no grids, no products), so the
oracle and the HIP library can both consume its outputs without sharing any of
the method's code.
"""
from .gen import (  # noqa: F401
    normal_f32,
    uniform_words,
    bf16_bits_from_f32,
    f32_from_bf16_bits,
    outlier_channels,
    activations_bf16,
    weights_f32,
    sample_rows,
)
from .workloads import LAYERS, DECODE_LAYERS, PREFILL_LAYERS, SHARD_LAYERS, Layer, config  # noqa: F401
