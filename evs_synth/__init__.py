"""Seeded synthetic workloads for the block-verify hot path.

This package holds the model shapes and the seeded generators of every input
(weights, prompts, draft distributions, uniforms, imported states). It holds
none of the method's arithmetic, so both the CPU oracle and the HIP library's
tests can draw the same inputs from it without sharing any computation.
"""
from .configs import Block, ModelConfig, tiny_c1, pair_c2, stack_7b, small_stack, drafter_1024, ACGT_IDS
from .gen import (make_weights, prompt_tokens, draft_probs_softmax, dirichlet_acgt,
                  uniforms, synthetic_state, rng_for, sample_from, weight_names, dyadic_weights)

__all__ = ["Block", "ModelConfig", "tiny_c1", "pair_c2", "stack_7b", "small_stack", "drafter_1024",
           "ACGT_IDS", "make_weights", "prompt_tokens", "draft_probs_softmax",
           "dirichlet_acgt", "uniforms", "synthetic_state", "rng_for", "sample_from",
           "weight_names", "dyadic_weights"]
