"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This package only draws random numbers, applies the token selection rule that produces the keep
mask, and runs the model's *forward* pass to produce the activations a backward pass consumes.
It holds none of the filtered-backward arithmetic: the oracle (``oracle/``) and the HIP library
(``token_filtered_backward_amd``) each implement that on their own, and neither imports the other.
"""
from .configs import CONFIGS, LayerShape, LinearShape, get_config  # noqa: F401
from .gen import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_keep,
    make_layer_inputs,
    make_linear_inputs,
    make_model_inputs,
    floats,
    suffix_keep,
    n_filtered,
    rng_for,
)
