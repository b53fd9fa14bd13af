"""Seeded synthetic inputs for the looped normalized-GPT forward pass.

This package holds the model shapes and the seeded generators of weights and
token ids. It is the only code shared by the oracle and the HIP path, and it
is shared as data: it holds none of the forward pass's arithmetic (no
attention, no update, no loop), only the recipe that draws the inputs.

Recipe (stated on the pages only as "random-init"; the details are ours):
weights are drawn N(0, 0.02) in float32 from a per-tensor PCG64 stream, then
scaled to unit L2 norm along the residual-stream (d_model) axis in float64,
then stored as float32 or as bfloat16 (round to nearest even). The nGPT
update weights (alpha) are filled with 0.05. Token ids are uniform over the
vocabulary.
"""
from .configs import ModelConfig, CONFIGS, get_config, scaled_config  # noqa: F401
from .gen import (  # noqa: F401
    make_weights,
    make_tokens,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    weight_names,
)
