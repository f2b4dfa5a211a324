"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This package only draws random numbers and rounds them to the storage dtype.
It holds none of the method's arithmetic (no scores, no selection, no attention).
"""
from .configs import CONFIGS, Config, config_by_name
from .generate import Inputs, LayerInputs, make_inputs, make_layer, make_resid_dout, to_bf16_bits_f32

__all__ = [
    "CONFIGS", "Config", "config_by_name",
    "Inputs", "LayerInputs", "make_inputs", "make_layer", "make_resid_dout", "to_bf16_bits_f32",
]
