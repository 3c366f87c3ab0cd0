"""Batches past 144 rows per launch: the rows are split into slices of whole
sequences, each launch normed once into bf16 rows. Each sequence of such a
batch must match the same sequence run alone bit for bit: block logits and,
after a ragged rollback, the committed state."""
import numpy as np
import pytest
import torch

import evs_synth as es
from evs_synth.configs import Block, ModelConfig
from oracle import HybridLM

from gpu_util import LOGIT_ATOL, logit_err, DEV, block_verify, lengths, prefill, rollback
from test_gpu_long_ragged import committed_equal
from attention_dna_lms_amd import evs

pytestmark = pytest.mark.gpu



def _engines(cfg, w, B, max_ctx, max_block=16):
    model = evs.Model(cfg, w, device=DEV)
    batch = evs.State(model, B, max_ctx, max_block, device=DEV)
    solo = [evs.State(model, 1, max_ctx, max_block, device=DEV) for _ in range(B)]
    return model, batch, solo


def _round_matches(cfg, model, batch, solo, cand, keep):
    B = cand.shape[0]
    lg, _ = block_verify(model, batch, cand)
    for b in range(B):
        one, _ = block_verify(model, solo[b], cand[b:b + 1])
        assert np.array_equal(one[0], lg[b]), b
    rollback(batch, keep)
    for b in range(B):
        rollback(solo[b], keep[b:b + 1])
    for b in range(B):
        assert committed_equal(cfg, batch, b, solo[b], 0), b
    return lg


def test_many_rows_small_stack_ragged_matches_solo():
    """The 8-layer stack (all mixer kinds), 14 sequences with prompts of 5..70
    tokens, two gamma = 12 rounds (182 rows: slices of 11 and 3 sequences),
    ragged rollbacks; sequence 0's first block also against the oracle."""
    cfg = es.small_stack()
    w = es.make_weights(cfg, seed=81)
    B, gamma = 14, 12
    rng = es.rng_for(82, "many-rows")
    plen = rng.integers(5, 71, B)
    prompts = [es.prompt_tokens(cfg, int(n), seed=83 + b)[0] for b, n in enumerate(plen)]
    model, batch, solo = _engines(cfg, w, B, 160)
    prefill(model, batch, prompts)
    for b in range(B):
        prefill(model, solo[b], [prompts[b]])
    for r in range(2):
        cand = es.prompt_tokens(cfg, gamma + 1, seed=90 + r, batch=B).astype(np.int32)
        keep = rng.integers(0, gamma + 2, B).astype(np.int32)
        lg = _round_matches(cfg, model, batch, solo, cand, keep)
        if r == 0:
            orc = HybridLM(cfg, w)
            _, ost = orc.prefill(prompts[0], chunk=16)
            assert logit_err(lg[0], orc.block(ost, cand[0]).logits) < LOGIT_ATOL
    assert np.array_equal(lengths(batch), np.array([lengths(s)[0] for s in solo]))
    assert batch.error() == 0 and all(s.error() == 0 for s in solo)


def test_many_rows_full_width_layers_match_solo():
    """d = 4096 layers (FIR-7, gated MLP 11008, attention 32 x 128, gated MLP),
    16 sequences x 13 candidates = 208 rows per launch."""
    cfg = ModelConfig("w4096_mix", 4096, 512, [Block("fir", fir_len=7), Block("mlp", d_ff=11008),
                                               Block("attn", n_heads=32, head_dim=128), Block("mlp", d_ff=11008)],
                      dtype="bf16")
    w = es.make_weights(cfg, seed=91, device=DEV)
    B, gamma = 16, 12
    prompts = [es.prompt_tokens(cfg, 24 + b, seed=92 + b)[0] for b in range(B)]
    model, batch, solo = _engines(cfg, w, B, 96)
    prefill(model, batch, prompts)
    for b in range(B):
        prefill(model, solo[b], [prompts[b]])
    cand = es.prompt_tokens(cfg, gamma + 1, seed=99, batch=B).astype(np.int32)
    keep = ((np.arange(B) * 5) % (gamma + 2)).astype(np.int32)
    _round_matches(cfg, model, batch, solo, cand, keep)
    assert batch.error() == 0
