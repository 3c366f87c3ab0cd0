"""Batched prefill (evs_prefill with several sequences: lockstep rounds of
max_block positions, prompts right-aligned) against per-sequence prefill:
the committed state, the last-token logits and the exported hidden rows are
equal bit for bit (block verify equals sequential decoding whatever the
chunking; model card, "Library": generation starts from a consumed prompt).
Ragged prompt lengths include an empty prompt, one shorter than a round,
exact multiples of the round and one longer than the others by a partial
round. The fp32 tiny stack and the bf16 8-layer stack; the bf16 case also
compares the last logits with the oracle's prefill.
"""
import numpy as np
import pytest
import torch

import evs_synth as es
from oracle import HybridLM

from gpu_util import DEV, LOGIT_ATOL, lengths, logit_err, storage_dtype
from test_gpu_long_ragged import committed_equal
from attention_dna_lms_amd import evs

pytestmark = pytest.mark.gpu


def run_prefill(model, state, prompts, export_block=None):
    cfg = model.cfg
    flat = np.concatenate([np.asarray(p, np.int32) for p in prompts])
    offs = np.concatenate([[0], np.cumsum([len(p) for p in prompts])]).astype(np.int32)
    last = torch.full((len(prompts), cfg.vocab), 7.0, dtype=storage_dtype(cfg), device=DEV)
    hid = None
    if export_block is not None:
        hid = torch.full((state.B * state.max_block * cfg.d_model,), 3.0, dtype=torch.float32, device=DEV)
        evs.evs_state_export(state, export_block, hid)
    evs.evs_prefill(model, state, torch.from_numpy(flat).to(DEV), offs, last)
    torch.cuda.synchronize()
    if export_block is not None:
        evs.evs_state_export(state, -1)
        hid = hid[:state.B * cfg.d_model].view(state.B, cfg.d_model)
    assert state.error() == 0
    return last, hid


@pytest.mark.parametrize("which", ["tiny_f32", "small_bf16"])
def test_batched_prefill_equals_per_sequence_prefill(which):
    cfg = es.tiny_c1() if which == "tiny_f32" else es.small_stack()
    w = es.make_weights(cfg, seed=401)
    model = evs.Model(cfg, w, device=DEV)
    mb = 16
    lens = [0, 5, 32, 16, 37, 1, 20, 33]   # 8 x 16 rows per round: the bf16 stack splits K
    prompts = [es.prompt_tokens(cfg, n, seed=402 + i)[0] if n else np.zeros(0, np.int32) for i, n in enumerate(lens)]
    export_block = len(cfg.blocks) - 2
    batch = evs.State(model, len(prompts), 256, mb, device=DEV)
    last_b, hid_b = run_prefill(model, batch, prompts, export_block)
    assert list(lengths(batch)) == lens
    for b, p in enumerate(prompts):
        solo = evs.State(model, 1, 256, mb, device=DEV)
        if len(p):
            last_s, hid_s = run_prefill(model, solo, [p], export_block)
            assert torch.equal(last_b[b], last_s[0]), b
            assert torch.equal(hid_b[b], hid_s[0]), b
        else:
            # an empty prompt leaves its rows untouched
            assert torch.all(last_b[b].float() == 7.0) and torch.all(hid_b[b] == 3.0)
        assert committed_equal(cfg, batch, b, solo, 0), b
    if which == "small_bf16":
        orc = HybridLM(cfg, w)
        for b, p in enumerate(prompts):
            if len(p) == 0:
                continue
            lg, _ = orc.prefill(p, chunk=mb)
            assert logit_err(last_b[b].double().cpu().numpy(), lg) < LOGIT_ATOL, b


def test_batched_prefill_then_block_verify_matches_per_sequence():
    """The state a batched prefill commits carries on: one block verify on
    the batch equals the same block on each sequence prefilled alone."""
    cfg = es.small_stack()
    w = es.make_weights(cfg, seed=411)
    model = evs.Model(cfg, w, device=DEV)
    lens, gamma = [23, 40, 9], 6
    prompts = [es.prompt_tokens(cfg, n, seed=412 + i)[0] for i, n in enumerate(lens)]
    cand = torch.as_tensor(es.prompt_tokens(cfg, gamma + 1, seed=415, batch=len(lens)), device=DEV)
    batch = evs.State(model, len(lens), 256, 16, device=DEV)
    run_prefill(model, batch, prompts)
    lg = torch.zeros(len(lens), gamma + 1, cfg.vocab, dtype=torch.bfloat16, device=DEV)
    evs.evs_block_verify(model, batch, cand, gamma, lg)
    torch.cuda.synchronize()
    for b, p in enumerate(prompts):
        solo = evs.State(model, 1, 256, 16, device=DEV)
        run_prefill(model, solo, [p])
        ls = torch.zeros(1, gamma + 1, cfg.vocab, dtype=torch.bfloat16, device=DEV)
        evs.evs_block_verify(model, solo, cand[b:b + 1].contiguous(), gamma, ls)
        torch.cuda.synchronize()
        assert torch.equal(lg[b], ls[0]), b
