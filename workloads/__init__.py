"""Seeded synthetic inputs for the dropless MoE layer workloads.

This module only draws and lays out inputs (random tensors, the per-expert
router bias, the cfg-5 logit construction and token mask).  It holds none of
the layer's own arithmetic: no routing, permutation, MLP or combine.  Both the
oracle tests and the GPU tests/bench take their inputs from here, and nothing
here imports either side.
"""
from .configs import CONFIGS, MoEConfig, get_config  # noqa: F401
from .gen import (  # noqa: F401
    make_router_inputs,
    make_expert_weights,
    make_tokens,
    bf16_bits,
    bits_to_float,
)
