"""Seeded synthetic inputs for the dropless MoE layer.

This package only draws random numbers and encodes them in the storage formats
the layer consumes (bf16 bit patterns, OCP e4m3 bytes with fp32 block scales).
It holds none of the layer's arithmetic: routing, permutation, the expert MLP
and the gradients live on each side (GPU library, CPU oracle) separately.
"""
from .gen import (CONFIGS, MoEInputs, make_inputs, make_config, make_prerouted_fp8, bf16_bits_from_f32,
                  e4m3_bits_from_f32, quantize_rows_1x128, quantize_blocks_128x128)

__all__ = ["CONFIGS", "MoEInputs", "make_inputs", "make_config", "make_prerouted_fp8", "bf16_bits_from_f32",
           "e4m3_bits_from_f32", "quantize_rows_1x128", "quantize_blocks_128x128"]
