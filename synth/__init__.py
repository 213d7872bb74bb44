"""Seeded synthetic inputs for the int4 expert-routed MoE layer.

This package only draws random numbers and stores them in the layer's storage
formats (bf16 bit patterns, packed 4-bit words). It holds none of the layer's
arithmetic, so both the fp64 oracle and the HIP path can take their inputs from
it without sharing any computation.
"""
from .moe_inputs import (  # noqa: F401
    Q4Weights,
    MoEInputs,
    CONFIGS,
    make_layer,
    make_config,
    redraw_token_rows,
)
