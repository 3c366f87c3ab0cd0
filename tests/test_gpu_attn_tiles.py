"""Blocks of more than 16 positions: attention runs their 16-query tiles in
pairs over one pass of the keys (an odd tile count pads the pair). Each
query's arithmetic must not depend on the tiles that share the pass, so a
block of P positions equals P single-position steps bit for bit, prefill in
chunks of P equals prefill in chunks of 16, and the block logits match the
oracle."""
import numpy as np
import pytest

import evs_synth as es
from oracle import HybridLM

from gpu_util import LOGIT_ATOL, logit_err, DEV, block_verify, lengths, make_engine, prefill, rollback
from attention_dna_lms_amd import evs

pytestmark = pytest.mark.gpu



@pytest.mark.parametrize("P,head_dim", [(17, 128), (32, 64), (40, 32), (40, 128)])
def test_query_tile_pairs_match_single_steps_and_oracle(P, head_dim):
    """The 8-layer stack (attention at layer 7) with 2-8 heads, two sequences
    with 50- and 37-token prompts, one block of P candidates each."""
    cfg = es.small_stack(head_dim=head_dim)
    w = es.make_weights(cfg, seed=200 + P + head_dim)
    prompts = [es.prompt_tokens(cfg, n, seed=201 + i)[0] for i, n in enumerate((50, 37))]
    cand = es.prompt_tokens(cfg, P, seed=203, batch=2).astype(np.int32)
    model, big = make_engine(cfg, w, batch=2, max_ctx=192, max_block=P)
    last_big = prefill(model, big, prompts)
    m16, small = make_engine(cfg, w, batch=2, max_ctx=192, max_block=16)
    last_small = prefill(m16, small, prompts)
    # prefill chunking (P against 16 positions per call) changes no bit
    assert np.array_equal(last_big, last_small)
    lg, _ = block_verify(model, big, cand)
    orc = HybridLM(cfg, w)
    for b in range(2):
        _, ost = orc.prefill(prompts[b], chunk=16)
        err = logit_err(lg[b], orc.block(ost, cand[b]).logits)
        assert err < LOGIT_ATOL, (b, err)
    # the same candidates one position per call, each committed before the next
    for k in range(P):
        one, _ = block_verify(m16, small, cand[:, k:k + 1])
        assert np.array_equal(one[:, 0], lg[:, k]), k
        rollback(small, [1, 1])
    assert list(lengths(small)) == [50 + P, 37 + P]
    assert big.error() == 0 and small.error() == 0
