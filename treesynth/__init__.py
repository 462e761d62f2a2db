"""Seeded synthetic inputs shared by the oracle and the HIP path.

This module only draws random numbers and lays out the trees it builds
itself: token sequences (rollouts that share prefixes) and dense input
tensors.  It holds none of the method's arithmetic -- it never computes a
DFS order, a mask, an attention output or a loss.  Both sides receive
exactly the same inputs from here; bf16 inputs are rounded once (RNE) here
so that the oracle sees the exact values the GPU sees.

Every generator uses numpy's PCG64 with an explicit seed.
"""
from .trees import (  # noqa: F401
    SynthTree,
    tiny_tree,
    rl_forest,
    rl_forest_accepted,
    agentic_beam_tree,
    long_chain,
    lmhead_tree,
    random_small_tree,
    nested_tree,
)
from .tensors import (  # noqa: F401
    rng_for,
    bf16_round,
    bf16_bits_to_f64,
    bf16_bits_to_f32,
    normal_f32,
    normal_bf16,
)
