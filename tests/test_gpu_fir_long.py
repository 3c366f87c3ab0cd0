"""FIR filters longer than the epilogue's register prefetch (> 128 taps) take
the generic window path: a 200-tap FIR with a gated MLP at d = 256, three
sequences in one launch, against the oracle and each sequence run alone."""
import numpy as np
import pytest

import evs_synth as es
from evs_synth.configs import Block, ModelConfig
from oracle import HybridLM

from gpu_util import LOGIT_ATOL, logit_err, DEV, block_verify, lengths, make_engine, prefill, rollback
from attention_dna_lms_amd import evs

pytestmark = pytest.mark.gpu



def test_fir_200_taps_batch_matches_oracle_and_single_sequences():
    cfg = ModelConfig("fir200_d256", 256, 512, [Block("fir", fir_len=200), Block("mlp", d_ff=672)], dtype="bf16")
    w = es.make_weights(cfg, seed=300)
    B, P = 3, 13
    plen = [30, 120, 250]                       # shorter than, near and longer than the window
    prompts = [es.prompt_tokens(cfg, n, seed=301 + b)[0] for b, n in enumerate(plen)]
    cand = es.prompt_tokens(cfg, P, seed=305, batch=B).astype(np.int32)
    model, state = make_engine(cfg, w, batch=B, max_ctx=320, max_block=16)
    prefill(model, state, prompts)
    lg, _ = block_verify(model, state, cand)
    keep = np.array([4, 13, 0], np.int32)
    rollback(state, keep)
    orc = HybridLM(cfg, w)
    for b in range(B):
        _, ost = orc.prefill(prompts[b], chunk=16)
        err = logit_err(lg[b], orc.block(ost, cand[b]).logits)
        assert err < LOGIT_ATOL, (b, err)
        m1, s1 = make_engine(cfg, w, batch=1, max_ctx=320, max_block=16)
        prefill(m1, s1, [prompts[b]])
        one, _ = block_verify(m1, s1, cand[b:b + 1])
        assert np.array_equal(one[0], lg[b]), b
        rollback(s1, keep[b:b + 1])
        assert lengths(s1)[0] == lengths(state)[b] == plen[b] + keep[b]
    assert state.error() == 0
