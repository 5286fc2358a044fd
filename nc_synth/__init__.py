"""Seeded synthetic inputs shared by the oracle and the GPU path.

This package holds the model configurations (shapes and scalar hyper-parameters
only) and the seeded generators for parameters and token batches.  It contains
none of the model's arithmetic: the oracle and the HIP library each implement
the forward and backward pass on their own, and both consume exactly the arrays
produced here.
"""
from .configs import CONFIGS, get_config, param_shapes
from .generators import (
    bf16_round,
    bf16_bits,
    bf16_from_bits,
    make_params,
    make_tokens,
    zipf_probs,
)

__all__ = [
    "CONFIGS", "get_config", "param_shapes", "bf16_round", "bf16_bits",
    "bf16_from_bits", "make_params", "make_tokens", "zipf_probs",
]
