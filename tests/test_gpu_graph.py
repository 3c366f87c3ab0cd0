"""A speculative round captured once as a HIP graph and replayed with
different per-sequence outcomes (Evo2 discussion #232, author reply, the
state-slicing contract, item 2: per-sequence accepted lengths in a batch, with
graph capture). Nothing in the captured round depends on the host: the
committed lengths, IIR buffer indices and slots live on the device, the
candidates and uniforms are read from fixed device buffers the host refills
between replays, and rollback keeps what the verifier decided.

Per replay the uniforms force each sequence to reject at a chosen position
(u = 0 accepts any draft with p > 0; u just below 1 rejects a draft whose
q is one-hot, since then p / q = p < 1), so n_keep sweeps 1 .. gamma + 1
across sequences and replays. Each replay is checked bit for bit against
the same round run eagerly on a twin state (logits, decisions, every
sequence's committed state), with eager work and synchronisations between
replays, and sequence 0's logits against the oracle, which follows it.
"""
import numpy as np
import pytest
import torch

import evs_synth as es
from oracle import HybridLM

from gpu_util import DEV, LOGIT_ATOL, lengths, logit_err, prefill
from test_gpu_long_ragged import committed_equal
from attention_dna_lms_amd import evs

pytestmark = pytest.mark.gpu

U_REJECT = np.float32(1.0) - np.float32(2.0 ** -24)      # largest fp32 below 1


def test_graph_replay_matches_eager_across_ragged_n_keep():
    cfg = es.small_stack()
    V = cfg.vocab
    w = es.make_weights(cfg, seed=81)
    B, gamma = 3, 6
    P = gamma + 1
    prompts = [es.prompt_tokens(cfg, n, seed=82 + b)[0] for b, n in enumerate((40, 23, 57))]
    model = evs.Model(cfg, w, device=DEV)
    sg = evs.State(model, B, 256, P, device=DEV)      # replayed
    se = evs.State(model, B, 256, P, device=DEV)      # eager twin
    prefill(model, sg, prompts)
    prefill(model, se, prompts)

    cand = torch.zeros(B, P, dtype=torch.int32, device=DEV)
    drafts = torch.zeros(B, gamma, dtype=torch.int32, device=DEV)      # cand[:, 1:], contiguous
    u = torch.zeros(B, P, dtype=torch.float32, device=DEV)
    q = torch.zeros(B, gamma, V, dtype=torch.float32, device=DEV)
    lg = torch.zeros(B, P, V, dtype=torch.bfloat16, device=DEV)
    acc = torch.zeros(B, dtype=torch.int32, device=DEV)
    nxt = torch.zeros(B, dtype=torch.int32, device=DEV)
    keep = torch.zeros(B, dtype=torch.int32, device=DEV)

    def round_on(state, cand, u, q, lg, acc, nxt, keep):
        evs.evs_block_verify(model, state, cand, gamma, lg)
        evs.evs_verify_sample(B, gamma, V, lg, evs.EVS_TARGET_LOGITS_BF16, q, drafts, u, 1.0, 0, 0,
                              acc, nxt, keep)
        evs.evs_rollback(state, keep)

    def fill(r):
        """Round r's inputs: candidates, one-hot q at each draft, and uniforms
        that make sequence b reject at position reject[b] (gamma: accept all)."""
        c = es.prompt_tokens(cfg, P, seed=90 + r, batch=B).astype(np.int32)
        reject = [(r + 3 * b) % (gamma + 1) for b in range(B)]
        uu = np.zeros((B, P), np.float32)
        for b, k in enumerate(reject):
            if k < gamma:
                uu[b, k] = U_REJECT
        uu[:, gamma] = es.uniforms((B,), seed=95 + r)
        qq = np.zeros((B, gamma, V), np.float32)
        for b in range(B):
            qq[b, np.arange(gamma), c[b, 1:]] = 1.0
        cand.copy_(torch.from_numpy(c))
        drafts.copy_(torch.from_numpy(np.ascontiguousarray(c[:, 1:])))
        u.copy_(torch.from_numpy(uu))
        q.copy_(torch.from_numpy(qq))
        return c, reject

    # capture (graph capture records without running; a warm-up round on the
    # capture stream first, on a scratch state, so nothing is allocated while capturing)
    scratch = evs.State(model, B, 256, P, device=DEV)
    prefill(model, scratch, prompts)
    fill(0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        round_on(scratch, cand, u, q, lg, acc, nxt, keep)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        round_on(sg, cand, u, q, lg, acc, nxt, keep)
    torch.cuda.synchronize()

    orc = HybridLM(cfg, w)
    _, ost = orc.prefill(prompts[0], chunk=64)
    lg_e = torch.zeros_like(lg)
    acc_e, nxt_e, keep_e = torch.zeros_like(acc), torch.zeros_like(nxt), torch.zeros_like(keep)
    seen = set()
    for r in range(6):
        c, reject = fill(r)
        t_before = lengths(se)
        graph.replay()
        torch.cuda.synchronize()
        round_on(se, cand, u, q, lg_e, acc_e, nxt_e, keep_e)
        torch.cuda.synchronize()
        assert torch.equal(lg, lg_e), r
        assert torch.equal(acc, acc_e) and torch.equal(nxt, nxt_e) and torch.equal(keep, keep_e), r
        k = keep.cpu().numpy()
        assert list(k) == [x + 1 for x in reject], (r, list(k), reject)
        seen.update(int(x) for x in k)
        assert np.array_equal(lengths(sg), t_before + k) and np.array_equal(lengths(se), t_before + k)
        for b in range(B):
            assert committed_equal(cfg, sg, b, se, b), (r, b)
        pend = orc.block(ost, c[0])
        assert logit_err(lg[0].double().cpu().numpy(), pend.logits) < LOGIT_ATOL, r
        ost = orc.rollback(pend, int(k[0]))
    assert seen == set(range(1, P + 1)), seen
    assert sg.error() == 0 and se.error() == 0
