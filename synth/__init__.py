"""Seeded synthetic inputs for the ResidualKV cache-write path.

This package only draws random numbers and lays them out; it holds none of the
method's arithmetic (no distances, no selection, no compressor, no quantiser).
Both the CPU oracle (``oracle/``) and the GPU library's tests and benchmark take
their inputs from here, so the two sides always see the same bits.
"""
from .configs import CONFIGS, RkvConfig, config_by_name
from .generate import (
    decoder_weight,
    Workload,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    generate,
)

__all__ = [
    "decoder_weight",
    "CONFIGS",
    "RkvConfig",
    "config_by_name",
    "Workload",
    "bf16_bits_to_f32",
    "f32_to_bf16_bits",
    "generate",
]
