"""evs_block_verify_noalloc (the workspace in the library's device scratch)
against evs_block_verify (the state's own workspace), through the C ABI: two
calls in a row, the second with a smaller block, each followed by a ragged
rollback. The two entry points run the same kernels in the same order, so
logits and every committed state must agree bit for bit (the bar for a
result that has one exact value). Also: the size limit and the state
without a workspace."""
import numpy as np
import pytest
import torch

import evs_synth as es
from oracle import HybridLM

from gpu_util import DEV, LOGIT_ATOL, lengths, logit_err, prefill
from test_gpu_long_ragged import committed_equal
from attention_dna_lms_amd import evs

pytestmark = pytest.mark.gpu


def test_noalloc_block_verify_equals_block_verify_two_calls():
    cfg = es.small_stack()
    V = cfg.vocab
    w = es.make_weights(cfg, seed=131)
    B, max_block = 3, 13
    prompts = [es.prompt_tokens(cfg, n, seed=132 + b)[0] for b, n in enumerate((45, 20, 61))]
    model = evs.Model(cfg, w, device=DEV)
    ref = evs.State(model, B, 256, max_block, device=DEV)
    nal = evs.State(model, B, 256, max_block, device=DEV, workspace=False)
    assert nal.ws is None and ref.workspace_bytes <= evs.EVS_NOALLOC_SCRATCH_BYTES
    prefill(model, ref, prompts)
    # the state without a workspace consumes its prompts through the no-alloc
    # block verify in chunks of max_block, keeping every position
    longest = max(len(p) for p in prompts)
    for a in range(0, longest, max_block):
        # every sequence advances by the same chunk; shorter prompts are padded
        # by repeating their last token and the padding is not kept
        P = min(max_block, longest - a)
        chunk = np.zeros((B, P), np.int32)
        keep = np.zeros(B, np.int32)
        for b, p in enumerate(prompts):
            n = max(0, min(P, len(p) - a))
            chunk[b, :n] = p[a:a + n]
            chunk[b, n:] = p[-1]
            keep[b] = n
        lg = torch.zeros(B, P, V, dtype=torch.bfloat16, device=DEV)
        evs.evs_block_verify_noalloc(model, nal, torch.from_numpy(chunk).to(DEV), P - 1, lg)
        evs.evs_rollback(nal, torch.from_numpy(keep).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(lengths(nal), lengths(ref))
    for b in range(B):
        assert committed_equal(cfg, nal, b, ref, b), b

    orc = HybridLM(cfg, w)
    ost = orc.prefill(prompts[0], chunk=64)[1]
    for r, gamma in enumerate((12, 4)):                 # the second call is smaller
        P = gamma + 1
        cand = torch.from_numpy(es.prompt_tokens(cfg, P, seed=140 + r, batch=B).astype(np.int32)).to(DEV)
        lg_ref = torch.zeros(B, P, V, dtype=torch.bfloat16, device=DEV)
        lg_nal = torch.full((B, P, V), float("nan"), dtype=torch.bfloat16, device=DEV)
        evs.evs_block_verify(model, ref, cand, gamma, lg_ref)
        evs.evs_block_verify_noalloc(model, nal, cand, gamma, lg_nal)
        torch.cuda.synchronize()
        assert torch.equal(lg_ref, lg_nal), r
        pend = orc.block(ost, cand[0].cpu().numpy())
        assert logit_err(lg_nal[0].double().cpu().numpy(), pend.logits) < LOGIT_ATOL, r
        keep = torch.tensor([(r + 2 * b) % (P + 1) for b in range(B)], dtype=torch.int32, device=DEV)
        t0 = lengths(ref)
        evs.evs_rollback(ref, keep)
        evs.evs_rollback(nal, keep)
        torch.cuda.synchronize()
        assert np.array_equal(lengths(nal), t0 + keep.cpu().numpy()) and np.array_equal(lengths(ref), lengths(nal))
        for b in range(B):
            assert committed_equal(cfg, nal, b, ref, b), (r, b)
        ost = orc.rollback(pend, int(keep[0]))
    assert ref.error() == 0 and nal.error() == 0


def test_noalloc_limits_and_workspace_free_state():
    cfg = es.small_stack()
    w = es.make_weights(cfg, seed=150)
    model = evs.Model(cfg, w, device=DEV)
    V = cfg.vocab
    # a state whose workspace exceeds the scratch: rejected before any launch
    big = evs.State(model, 64, 256, 64, device=DEV, workspace=False)
    assert big.workspace_bytes > evs.EVS_NOALLOC_SCRATCH_BYTES
    cand = torch.zeros(64, 2, dtype=torch.int32, device=DEV)
    lg = torch.zeros(64, 2, V, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(evs.EvsError) as e:
        evs.evs_block_verify_noalloc(model, big, cand, 1, lg)
    assert e.value.status == -2                          # EVS_E_RANGE
    # a state without a workspace: the calls that need one refuse it
    nal = evs.State(model, 1, 256, 8, device=DEV, workspace=False)
    with pytest.raises(evs.EvsError) as e:
        evs.evs_block_verify(model, nal, cand[:1], 1, lg[:1])
    assert e.value.status == -3                          # EVS_E_STATE
    with pytest.raises(evs.EvsError) as e:
        evs.evs_prefill(model, nal, cand[:1].view(-1), [0, 2], None)
    assert e.value.status == -3
    assert lengths(nal)[0] == 0 and nal.error() == 0
