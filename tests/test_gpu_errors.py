"""Device-side error handling: conditions only the device sees are clamped in
bounds and set a bit of the state's sticky error word (token ids out of range,
a block running past the context capacity, a device n_keep outside 0..P, draft
ids out of range). Each case is checked against the equivalent valid call."""
import numpy as np
import pytest
import torch

import evs_synth as es

from gpu_util import DEV, block_verify, lengths, make_engine, prefill, rollback
from attention_dna_lms_amd import evs

pytestmark = pytest.mark.gpu

ERR_TOKEN, ERR_CONTEXT, ERR_NKEEP, ERR_DRAFT = 1, 2, 4, 8


def _engine(max_ctx=512):
    cfg = es.small_stack()
    w = es.make_weights(cfg, seed=41)
    prompt = es.prompt_tokens(cfg, 60, seed=42)[0]
    model, state = make_engine(cfg, w, batch=1, max_ctx=max_ctx, max_block=16)
    prefill(model, state, [prompt])
    assert state.error(clear=True) == 0
    return cfg, model, state


def test_token_out_of_range_reads_as_token_zero():
    cfg, model, state = _engine()
    snap = state.buf.clone()
    cand = es.prompt_tokens(cfg, 13, seed=43)[0].copy()
    good = cand.copy()
    good[4] = 0
    ref, _ = block_verify(model, state, good[None])
    assert state.error(clear=True) == 0
    state.buf.copy_(snap)
    cand[4] = cfg.vocab + 7
    lg, _ = block_verify(model, state, cand[None])
    assert state.error(clear=True) == ERR_TOKEN
    assert np.array_equal(lg, ref)


def test_block_past_capacity_is_flagged():
    cfg, model, state = _engine(max_ctx=64)          # 60 committed + 13 > 64
    cand = es.prompt_tokens(cfg, 13, seed=44)[0]
    block_verify(model, state, cand[None])
    assert state.error(clear=True) & ERR_CONTEXT
    rollback(state, [0])                             # nothing kept: the committed state is untouched
    assert list(lengths(state)) == [60]


def test_device_n_keep_out_of_range_is_clamped():
    cfg, model, state = _engine()
    cand = es.prompt_tokens(cfg, 13, seed=45)[0]
    block_verify(model, state, cand[None])
    rollback(state, [13 + 5])                        # more than the block: clamped to 13
    assert state.error(clear=True) == ERR_NKEEP
    assert list(lengths(state)) == [73]
    block_verify(model, state, cand[None])
    rollback(state, [-3])                            # negative: clamped to 0
    assert state.error(clear=True) == ERR_NKEEP
    assert list(lengths(state)) == [73]


def test_draft_id_out_of_range_is_clamped_and_flagged():
    B, gamma, V = 2, 4, 512
    rng = np.random.default_rng(46)
    logits = torch.from_numpy(rng.normal(0, 1, (B, gamma + 1, V)).astype(np.float32)).to(torch.bfloat16).to(DEV)
    lf = logits.float().cpu().numpy()
    drafts = lf[:, :gamma].argmax(-1).astype(np.int32)
    drafts[1, 2] = V + 100                            # clamped to V - 1
    out = []
    for dr in (drafts, np.where(drafts >= V, V - 1, drafts).astype(np.int32)):
        n_acc = torch.zeros(B, dtype=torch.int32, device=DEV)
        nxt = torch.zeros(B, dtype=torch.int32, device=DEV)
        keep = torch.zeros(B, dtype=torch.int32, device=DEV)
        err = torch.zeros(1, dtype=torch.int32, device=DEV)
        evs.evs_verify_sample(B, gamma, V, logits, evs.EVS_TARGET_LOGITS_BF16, None, torch.as_tensor(dr).to(DEV),
                              None, 1.0, 0, 1, n_acc, nxt, keep, err)
        torch.cuda.synchronize()
        out.append((n_acc.cpu().numpy(), nxt.cpu().numpy(), int(err[0])))
    assert out[0][2] == ERR_DRAFT and out[1][2] == 0
    assert np.array_equal(out[0][0], out[1][0]) and np.array_equal(out[0][1], out[1][1])
    assert out[0][0][0] == gamma and out[0][0][1] == 2
