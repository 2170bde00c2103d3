"""Seeded synthetic inputs for the tensor-parallel MLP / attention-projection shard.

This package is the only code shared by the CPU oracle (``oracle/``) and the HIP
path (``tensor_transformer_layer_fwd_amd/``). It holds the five workload shapes
and the seeded random draws, and nothing of the method's arithmetic: no matrix
product, no activation, no sum over shards.
"""
from .configs import CONFIGS, TPConfig, get_config
from .generate import (
    INPUT_ORDER,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_inputs,
)

__all__ = [
    "CONFIGS",
    "TPConfig",
    "get_config",
    "INPUT_ORDER",
    "make_inputs",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
]
