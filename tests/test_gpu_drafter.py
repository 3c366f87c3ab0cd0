"""GPU parity of the drafter path: the target's hidden-state export, the
drafter's injected prefix, slots, trunk and head (evs_draft) against the
oracle drafter, the Markov draws bit for bit on the same logits, the exact
causal prefix, and the device-side index check."""
import numpy as np
import pytest
import torch

import evs_synth as es
from oracle import HybridLM
from oracle.drafter import Drafter

from gpu_util import LOGIT_ATOL, logit_err, DEV, block_verify, make_engine, prefill, rollback
from attention_dna_lms_amd import evs

pytestmark = pytest.mark.gpu



def test_hidden_export_matches_oracle_and_sequential_steps():
    """Residual rows after block 11 (layer 5's MLP) of the 8-layer stack,
    exported during a 13-candidate block verify: against the oracle's block
    form, and bit for bit against the same rows exported by 13 single-token
    verifies (the forward is batch invariant)."""
    cfg = es.small_stack()
    w = es.make_weights(cfg, seed=51)
    prompt = es.prompt_tokens(cfg, 40, seed=52)[0]
    cand = es.prompt_tokens(cfg, 13, seed=53)[0]
    blk = 11
    model, state = make_engine(cfg, w, batch=1, max_ctx=128, max_block=16)
    prefill(model, state, [prompt])
    dst = torch.full((1, 16, cfg.d_model), float("nan"), device=DEV)
    evs.evs_state_export(state, blk, dst)
    block_verify(model, state, cand[None])
    ex = dst[0, :13].double().cpu().numpy()
    orc = HybridLM(cfg, w)
    _, ost = orc.prefill(prompt, chunk=16)
    ref = orc.block(ost, cand, keep_x=True).x_out[blk]
    assert np.max(np.abs(ex - ref)) < LOGIT_ATOL * max(1.0, float(np.max(np.abs(ref)))), np.max(np.abs(ex - ref))
    m2, s2 = make_engine(cfg, w, batch=1, max_ctx=128, max_block=16)
    prefill(m2, s2, [prompt])
    one = torch.full((1, 16, cfg.d_model), float("nan"), device=DEV)
    evs.evs_state_export(s2, blk, one)
    for k in range(13):
        block_verify(m2, s2, cand[None, k:k + 1])
        assert torch.equal(one[0, 0], dst[0, k]), k
        rollback(s2, [1])
    evs.evs_state_export(s2, -1)
    assert state.error() == 0 and s2.error() == 0


def _drafter(seed=61, B=2):
    cfg = es.drafter_1024()
    w = es.make_weights(cfg, seed=seed)
    model = evs.Model(cfg, w, device=DEV)
    state = evs.State(model, B, cfg.max_slots, cfg.max_slots, device=DEV)
    torch.cuda.synchronize()
    return cfg, w, model, state


def _hidden(B, rows, K, seed):
    h = es.rng_for(seed, "hidden").standard_normal((B, rows, K)).astype(np.float32)
    h[1] *= 1e11                 # the residual scale the pages report for the last target blocks
    return h


def _run(model, state, B, h, idx, last, gamma, u, T, top_k, greedy):
    V = model.cfg.vocab
    lg = torch.empty(B, gamma, V, dtype=torch.bfloat16, device=DEV)
    dr = torch.full((B, gamma), -7, dtype=torch.int32, device=DEV)
    q = torch.full((B, gamma, V), float("nan"), device=DEV)
    evs.evs_draft(model, state, B, torch.as_tensor(h).to(DEV), h.shape[1],
                  None if idx is None else torch.as_tensor(np.asarray(idx, np.int32)).to(DEV),
                  torch.as_tensor(np.asarray(last, np.int32)).to(DEV), gamma,
                  None if u is None else torch.as_tensor(u).to(DEV), T, top_k, greedy, lg, dr, q)
    torch.cuda.synchronize()
    return lg.double().cpu().numpy(), dr.cpu().numpy(), q.cpu().numpy()


def test_drafter_matches_oracle_and_draws_bitexact():
    """d = 1024 drafter (one attention 8 x 128 + gated-MLP layer), a 4096-wide
    injected prefix (one sequence's hidden row at 1e11 scale), gamma = 12:
    head logits against the oracle drafter; drafts and q bit for bit against
    the oracle's Markov head and draws on the GPU's own logits (sampling at
    T = 1 with top-4, and greedy)."""
    B, gamma = 2, 12
    cfg, w, model, state = _drafter()
    h = _hidden(B, 3, cfg.inject_dim, 62)
    idx, last = [2, 0], [65, 84]
    u = es.uniforms((B, gamma), seed=63)
    lg, dr, q = _run(model, state, B, h, idx, last, gamma, u, 1.0, 4, 0)
    orc = Drafter(cfg, w)
    for b in range(B):
        ref = orc.trunk_logits(h[b, idx[b]].astype(np.float64), last[b], gamma)
        err = logit_err(lg[b], ref)
        assert err < LOGIT_ATOL, (b, err)
        d_ref, q_ref = orc.draft(lg[b], last[b], u[b], 1.0, 4)
        assert np.array_equal(dr[b], d_ref), b
        assert np.array_equal(q[b], q_ref), b
    lg2, dr2, _ = _run(model, state, B, h, idx, last, gamma, None, 1.0, 0, 1)
    assert np.array_equal(lg2, lg)
    for b in range(B):
        d_ref, _ = orc.draft(lg2[b], last[b], greedy=True)
        assert np.array_equal(dr2[b], d_ref), b
    assert state.error() == 0


@pytest.mark.parametrize("T,top_k", [(1.0, 1), (0.7, 16), (1.3, 17), (1.0, 0), (0.5, 5)])
def test_drafter_draws_bitexact_over_top_k(T, top_k):
    """Drafts and q bit for bit against the oracle's Markov head and draws on
    the GPU's logits across the kept-set paths: top-k up to 16 (the kept
    entries alone), beyond 16 and no cut (the full row)."""
    B, gamma = 3, 12
    cfg, w, model, state = _drafter(seed=69, B=B)
    h = _hidden(B, 2, cfg.inject_dim, 70)
    idx, last = [1, 0, 1], [65, 67, 71]
    u = es.uniforms((B, gamma), seed=71 + top_k)
    u[2, 3] = 0.0
    lg, dr, q = _run(model, state, B, h, idx, last, gamma, u, T, top_k, 0)
    orc = Drafter(cfg, w)
    for b in range(B):
        d_ref, q_ref = orc.draft(lg[b], last[b], u[b], T, top_k)
        assert np.array_equal(dr[b], d_ref), (b, dr[b], d_ref)
        assert np.array_equal(q[b], q_ref), b
    _, dg, qg = _run(model, state, B, h, idx, last, gamma, None, T, top_k, 1)
    for b in range(B):
        d_ref, q_ref = orc.draft(lg[b], last[b], None, T, top_k, greedy=True)
        assert np.array_equal(dg[b], d_ref), b
        assert np.array_equal(qg[b], q_ref), b
    assert state.error() == 0


@pytest.mark.parametrize("top_k", [4, 0])
def test_drafter_large_vocab_row_path(top_k):
    """A vocabulary past 512 takes the kernel that keeps the row in LDS: a
    small drafter (d = 128, V = 600) against the oracle drafter, draws bit
    for bit on the GPU's logits."""
    from evs_synth.configs import Block, ModelConfig
    cfg = ModelConfig("drafter_v600", 128, 600, [Block("attn", n_heads=4, head_dim=32), Block("mlp", d_ff=352)],
                      dtype="bf16", inject_dim=96, max_slots=8)
    w = es.make_weights(cfg, seed=72)
    B, gamma = 2, 8
    model = evs.Model(cfg, w, device=DEV)
    state = evs.State(model, B, 8, 8, device=DEV)
    h = _hidden(B, 1, cfg.inject_dim, 73)
    u = es.uniforms((B, gamma), seed=74)
    lg, dr, q = _run(model, state, B, h, None, [65, 599], gamma, u, 0.9, top_k, 0)
    orc = Drafter(cfg, w)
    for b, last in enumerate([65, 599]):
        ref = orc.trunk_logits(h[b, 0].astype(np.float64), last, gamma)
        assert logit_err(lg[b], ref) < LOGIT_ATOL
        d_ref, q_ref = orc.draft(lg[b], last, u[b], 0.9, top_k)
        assert np.array_equal(dr[b], d_ref), b
        assert np.array_equal(q[b], q_ref), b
    assert state.error() == 0


def test_drafter_exact_causal_prefix_on_gpu():
    """A shorter draft is an exact prefix of a longer one: logits rows and
    drafts of gamma = 5 equal the first 5 of gamma = 12 bit for bit."""
    B = 2
    cfg, w, model, state = _drafter(seed=64)
    h = _hidden(B, 1, cfg.inject_dim, 65)
    u = es.uniforms((B, 12), seed=66)
    lg12, d12, q12 = _run(model, state, B, h, None, [71, 67], 12, u, 0.8, 0, 0)
    lg5, d5, q5 = _run(model, state, B, h, None, [71, 67], 5, u[:, :5].copy(), 0.8, 0, 0)
    assert np.array_equal(lg12[:, :5], lg5)
    assert np.array_equal(d12[:, :5], d5)
    assert np.array_equal(q12[:, :5], q5)


def test_hidden_index_out_of_range_is_clamped_and_flagged():
    B = 2
    cfg, w, model, state = _drafter(seed=67)
    h = _hidden(B, 3, cfg.inject_dim, 68)
    a = _run(model, state, B, h, [5, -1], [65, 65], 4, None, 1.0, 0, 1)
    assert state.error(clear=True) == evs.EVS_ERR_INDEX
    b = _run(model, state, B, h, [2, 0], [65, 65], 4, None, 1.0, 0, 1)
    assert state.error() == 0
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
