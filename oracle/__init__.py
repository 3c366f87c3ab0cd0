"""CPU oracle for the EvSpark block-verify hot path — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct NumPy implementation of what the path
computes, used to check the HIP library. Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import it; the product path never
does, and it shares no code with the HIP library (both only draw inputs from
the seeded generators in ``evs_synth``).

Contents
  numerics  — bf16 round-to-nearest-even, exact-erf GELU, RMSNorm (fp64).
  hybrid    — the hybrid stack: sequential single-token decoding (the
              definition), the block-verification forward over gamma+1
              candidates with per-position state, and state slicing.
  verifier  — exact rejection-sampling and greedy verification (fp32, the
              precision the GPU decides in).
  spec      — one speculative round and the snapshot-and-replay reference.
  drafter   — the gamma-parallel drafter: hidden-state prefix, trunk, Markov
              head and the sequential draws.
  fp8       — the FP8 (E4M3) weight variant's quantiser.

Precision: fp64 throughout, with values rounded to the model's storage type at
the points the bf16 path stores them (projection outputs, mixer outputs, KV
rows, MLP hidden, logits); fp32 models store without rounding. The verifier
runs in fp32 with every sum taken sequentially in index order, since its
floating-point results decide integers (accept counts and tokens).

Parity status per function is listed in each module's header.
"""
from .numerics import round_bf16, gelu, rmsnorm
from .hybrid import HybridLM, SeqState, Pending, fir_conv, iir_scan, causal_attention
from .verifier import target_probs, verify_sample, verify_greedy, icdf
from .spec import spec_round, native_greedy, replay
from .drafter import Drafter

__all__ = ["round_bf16", "gelu", "rmsnorm", "HybridLM", "SeqState", "Pending", "fir_conv",
           "iir_scan", "causal_attention",
           "target_probs", "verify_sample", "verify_greedy", "icdf", "spec_round",
           "native_greedy", "replay", "Drafter"]
