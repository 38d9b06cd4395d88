"""Seeded synthetic workloads shared by the tests, the bench and the smoke run.

This package only describes inputs: the arena shapes of the models the pages
train and seeded random gradients and weights of those shapes.  It holds none
of the pipeline's arithmetic (no reduction, norm, optimizer or rounding), so
both the GPU path and the CPU oracle can be fed from it without sharing code.
"""

from .shapes import ARENAS, Arena, arena, char_gpt, gpt2, llama
from .synth import (GRAD_SEED, grad_seed, master_init, onerank_inputs, peer_partials,
                    rank_grad, to_bits)

__all__ = ["ARENAS", "Arena", "arena", "char_gpt", "gpt2", "llama", "GRAD_SEED",
           "grad_seed", "master_init", "onerank_inputs", "peer_partials", "rank_grad",
           "to_bits"]
