"""GPU parity of the FP8 (E4M3) weight variant: block projections quantised at
packing with per-row power-of-two scales, bf16 activations, fp32 accumulation.
The oracle runs the same model with the FP8 effective weights q * s."""
import numpy as np
import pytest
import torch

import evs_synth as es
from evs_synth.configs import Block, ModelConfig
from oracle import HybridLM
from oracle.fp8 import fp8_weights

from gpu_util import LOGIT_ATOL, logit_err, DEV, block_verify, lengths, prefill, rollback, snapshot
from attention_dna_lms_amd import evs

pytestmark = pytest.mark.gpu



def engine(cfg, w, fp8, batch=1, max_ctx=256, max_block=16):
    model = evs.Model(cfg, w, device=DEV, fp8_weights=fp8)
    state = evs.State(model, batch, max_ctx, max_block, device=DEV)
    torch.cuda.synchronize()
    return model, state


def test_fp8_dyadic_layer_equals_bf16_bitexact():
    """Dyadic weights n * 2^-8 (|n| <= 4) quantise exactly (row scales 2^-14
    .. 2^-16 turn them into multiples of 64 that E4M3 holds), and at K = 4096
    the FP8 launch splits K over the waves as the bf16 one does: the FP8 model
    must reproduce the bf16 model bit for bit (logits and the FIR state)."""
    cfg = ModelConfig("fir7_d4096", 4096, 512, [Block("fir", fir_len=7)], dtype="bf16")
    w = es.dyadic_weights(cfg, seed=31)
    prompt = es.prompt_tokens(cfg, 40, seed=32)[0]
    cand = es.prompt_tokens(cfg, 13, seed=33)[0]
    out = []
    for fp8 in (False, True):
        m, s = engine(cfg, w, fp8)
        last = prefill(m, s, [prompt])
        lg, _ = block_verify(m, s, cand[None])
        rollback(s, [9])
        out.append((last, lg, snapshot(s, cfg)))
    assert np.array_equal(out[0][0], out[1][0])
    assert np.array_equal(out[0][1], out[1][1])
    assert np.array_equal(out[0][2]["fir"][0], out[1][2]["fir"][0])
    orc = HybridLM(cfg, fp8_weights(cfg, w))
    _, ost = orc.prefill(prompt, chunk=16)
    assert logit_err(out[1][1][0], orc.block(ost, cand).logits) < LOGIT_ATOL


def test_fp8_full_width_layers_match_oracle_and_steps():
    """A 7B-width FIR mixer and gated MLP (d = 4096, d_ff = 11008) with normal
    random-init weights: FP8 block logits against the oracle run on the FP8
    effective weights, and the FP8 block equal to 13 single steps bit for bit."""
    cfg = ModelConfig("fir_mlp_d4096", 4096, 512, [Block("fir", fir_len=7), Block("mlp", d_ff=11008)], dtype="bf16")
    w = es.make_weights(cfg, seed=34)
    P = 13
    prompt = es.prompt_tokens(cfg, 40, seed=35)[0]
    cand = es.prompt_tokens(cfg, P, seed=36)[0]
    mA, sA = engine(cfg, w, True)
    prefill(mA, sA, [prompt])
    blk, _ = block_verify(mA, sA, cand[None])
    print("fp8: oracle", flush=True)
    orc = HybridLM(cfg, fp8_weights(cfg, w))
    _, ost = orc.prefill(prompt, chunk=16)
    err = logit_err(blk[0], orc.block(ost, cand).logits)
    assert err < LOGIT_ATOL, err
    mB, sB = engine(cfg, w, True)
    prefill(mB, sB, [prompt])
    for k in range(P):
        one, _ = block_verify(mB, sB, cand[None, k:k + 1])
        assert np.array_equal(one[0, 0], blk[0, k]), k
        rollback(sB, [1])
    assert list(lengths(sB)) == [40 + P]


def test_fp8_batch_equals_single_sequences():
    """Four sequences in one FP8 launch (52 rows: the gate/up and in-projection
    norm fused into the GEMM prologue) against each run alone (13 rows: the
    single-tile gate/up over the norm kernel's bf16 rows): logits and, after a
    ragged rollback, lengths bit for bit. The two operand paths form the same
    bf16(x * rinv)."""
    cfg = ModelConfig("fir_mlp_d4096", 4096, 512, [Block("fir", fir_len=7), Block("mlp", d_ff=11008)], dtype="bf16")
    w = es.make_weights(cfg, seed=37)
    B, P = 4, 13
    prompts = [es.prompt_tokens(cfg, 20 + 7 * b, seed=38 + b)[0] for b in range(B)]
    cand = es.prompt_tokens(cfg, P, seed=43, batch=B).astype(np.int32)
    mA, sA = engine(cfg, w, True, batch=B)
    prefill(mA, sA, prompts)
    blk, _ = block_verify(mA, sA, cand)
    keep = np.array([0, 5, 13, 9], np.int32)
    rollback(sA, keep)
    for b in range(B):
        mB, sB = engine(cfg, w, True)
        prefill(mB, sB, [prompts[b]])
        one, _ = block_verify(mB, sB, cand[b:b + 1])
        assert np.array_equal(one[0], blk[b]), b
        rollback(sB, keep[b:b + 1])
        assert lengths(sB)[0] == lengths(sA)[b], b
    assert sA.error() == 0
