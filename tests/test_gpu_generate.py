"""The generation loop over the C ABI (evs_generate; model card, "Library":
generate and generate_native, speculative greedy output equal to native
output token for token) against the oracle's chained rounds
(oracle.spec.generate) with the same uniforms:
  * fp32 tiny stack with a random-init fp32 drafter model, sampling (T = 1 and
    T = 0.8 / top-3): every emitted id, the round count and the tokens per
    round equal the oracle's;
  * fp32 tiny stack, native decoding, greedy and sampled: equal to the oracle;
  * bf16 8-layer stack, greedy: the identity drafter (the native continuation
    as the proposal table) accepts every draft, a corrupted drafter (a quarter
    of the slots replaced by a random DNA letter) emits the same ids,
    both equal to native decoding through the same loop; the committed length
    after generation is the prompt plus every emitted token but the last;
  * too few rounds for n_tokens: EVS_E_RANGE with what was emitted so far.
"""
import numpy as np
import pytest
import torch

import evs_synth as es
from evs_synth.configs import ACGT_IDS, Block, ModelConfig
from oracle import HybridLM
from oracle.drafter import Drafter
from oracle.spec import generate as oracle_generate

from gpu_util import DEV, lengths
from attention_dna_lms_amd import evs

pytestmark = pytest.mark.gpu


def tiny_drafter_f32(vocab=4, inject_dim=128):
    return ModelConfig("tiny_drafter_f32", 64, vocab, [Block("attn", n_heads=2, head_dim=32), Block("mlp", d_ff=128)],
                       dtype="f32", inject_dim=inject_dim, max_slots=8)


@pytest.mark.parametrize("T,top_k", [(1.0, 0), (0.8, 3)])
def test_sampled_generation_with_a_drafter_model_equals_oracle(T, top_k):
    cfg = es.tiny_c1()
    w = es.make_weights(cfg, seed=201)
    dcfg = tiny_drafter_f32()
    dw = es.make_weights(dcfg, seed=202)
    B, gamma, n, export_block = 2, 4, 24, 3
    prompts = [es.prompt_tokens(cfg, L, seed=203 + b)[0] for b, L in enumerate((33, 20))]
    cap = n
    u_first = es.uniforms((B,), seed=205)
    u_t = es.uniforms((cap, B, gamma + 1), seed=206)
    u_d = es.uniforms((cap, B, gamma), seed=207)
    model = evs.Model(cfg, w, device=DEV)
    state = evs.State(model, B, 256, 16, device=DEV)
    dmodel = evs.Model(dcfg, dw, device=DEV)
    dstate = evs.State(dmodel, B, 64, 8, device=DEV)
    res = evs.generate(model, state, prompts, n, gamma=gamma, temperature=T, top_k=top_k, drafter=dmodel,
                       drafter_state=dstate, export_block=export_block, u_first=u_first, u_target=u_t, u_draft=u_d)
    orc, dr = HybridLM(cfg, w), Drafter(dcfg, dw)
    for b in range(B):
        ids, rounds, em = oracle_generate(orc, prompts[b], n, gamma, temperature=T, top_k=top_k, u_first=u_first[b],
                                          u_target=u_t[:, b], drafter=dr, export_block=export_block,
                                          u_draft=u_d[:, b], prefill_chunk=16)
        assert np.array_equal(res.ids[b], ids), (b, res.ids[b], ids)
        assert tuple(res.stats[b]) == (rounds, em), (b, tuple(res.stats[b]), (rounds, em))
    assert res.rounds == res.stats[:, 0].max()
    assert list(lengths(state)) == [len(p) + n - 1 for p in prompts]
    assert state.error() == 0 and dstate.error() == 0


@pytest.mark.parametrize("greedy", [True, False])
def test_native_generation_equals_oracle(greedy):
    cfg = es.tiny_c1()
    w = es.make_weights(cfg, seed=211)
    B, n = 3, 30
    prompts = [es.prompt_tokens(cfg, L, seed=212 + b)[0] for b, L in enumerate((17, 40, 9))]
    u_first = es.uniforms((B,), seed=215)
    u_t = es.uniforms((n, B, 1), seed=216)
    model = evs.Model(cfg, w, device=DEV)
    state = evs.State(model, B, 128, 8, device=DEV)
    res = evs.generate_native(model, state, prompts, n, greedy=greedy, temperature=1.0, top_k=0, u_first=u_first,
                              u_target=u_t)
    orc = HybridLM(cfg, w)
    for b in range(B):
        ids, rounds, _ = oracle_generate(orc, prompts[b], n, 0, greedy=greedy, u_first=u_first[b],
                                         u_target=u_t[:, b], prefill_chunk=8)
        assert np.array_equal(res.ids[b], ids), b
        assert res.stats[b, 0] == rounds == n - 1
    assert res.mean_tau == 1.0 and res.rounds == n - 1


def test_greedy_speculative_generation_equals_native_bf16():
    cfg = es.small_stack()
    w = es.make_weights(cfg, seed=221)
    B, gamma, n = 2, 12, 48
    prompts = [es.prompt_tokens(cfg, L, seed=222 + b)[0] for b, L in enumerate((50, 31))]
    model = evs.Model(cfg, w, device=DEV)

    def run(**kw):
        state = evs.State(model, B, 256, gamma + 1, device=DEV)
        res = evs.generate(model, state, prompts, n, greedy=True, **kw)
        assert list(lengths(state)) == [len(p) + n - 1 for p in prompts]
        assert state.error() == 0
        return res

    nat = run(gamma=0)
    assert nat.rounds == n - 1
    # identity drafter: the native continuation as the proposals
    table = np.concatenate([nat.ids, np.repeat(nat.ids[:, -1:], gamma, axis=1)], axis=1)
    ide = run(gamma=gamma, table=table)
    assert np.array_equal(ide.ids, nat.ids)
    # every round but the last accepts all gamma drafts (the last one's drafts
    # run past the table's n_tokens and are cut anyway)
    assert ide.rounds == -(-(n - 1) // (gamma + 1))
    assert np.all(ide.stats[:, 1] >= (gamma + 1) * (ide.rounds - 1) + 1) and np.all(ide.stats[:, 0] == ide.rounds)
    # a corrupted drafter: each slot independently replaced (p = 0.25) by a
    # uniformly drawn DNA letter (which may happen to be the right one)
    rng = es.rng_for(225, "replace")
    acgt = np.asarray(ACGT_IDS(cfg.vocab))
    rep = np.where(rng.random((n, B, gamma)) < 0.25, acgt[rng.integers(0, 4, (n, B, gamma))], -1)
    d75 = run(gamma=gamma, table=table, replace=rep)
    assert np.array_equal(d75.ids, nat.ids)
    assert d75.rounds >= 3 and d75.rounds > ide.rounds
    assert 1.0 < d75.mean_tau < gamma + 1


def test_too_few_rounds_is_a_range_error():
    cfg = es.tiny_c1()
    w = es.make_weights(cfg, seed=231)
    model = evs.Model(cfg, w, device=DEV)
    state = evs.State(model, 1, 128, 8, device=DEV)
    with pytest.raises(evs.EvsError) as e:
        evs.generate_native(model, state, [es.prompt_tokens(cfg, 12, seed=232)[0]], 10, greedy=True, rounds_cap=4)
    assert e.value.status == -2
    assert lengths(state)[0] == 12 + 4                  # the prompt and the four rounds' tokens


def test_greedy_corrupted_drafter_equals_oracle_native_greedy():
    """fp32 tiny stack, gamma = 6: the native continuation as the proposal
    table with a quarter of the slots replaced by random letters; the emitted
    ids equal the oracle's native greedy decoding (oracle.spec.native_greedy
    after the first argmax) over several rounds."""
    from oracle.spec import native_greedy
    from oracle.verifier import argmax_lowest
    cfg = es.tiny_c1()
    w = es.make_weights(cfg, seed=241)
    B, gamma, n = 2, 6, 36
    prompts = [es.prompt_tokens(cfg, L, seed=242 + b)[0] for b, L in enumerate((25, 44))]
    orc = HybridLM(cfg, w)
    want = []
    for p in prompts:
        lg, st = orc.prefill(p, chunk=8)
        first = argmax_lowest(lg)
        cont, _ = native_greedy(orc, st, first, n - 1)
        want.append(np.concatenate([[first], cont]))
    want = np.stack(want)
    table = np.concatenate([want, np.repeat(want[:, -1:], gamma, axis=1)], axis=1)
    rng = es.rng_for(245, "replace")
    rep = np.where(rng.random((n, B, gamma)) < 0.25, rng.integers(0, 4, (n, B, gamma)), -1)
    model = evs.Model(cfg, w, device=DEV)
    state = evs.State(model, B, 128, 8, device=DEV)
    res = evs.generate(model, state, prompts, n, gamma=gamma, greedy=True, table=table, replace=rep)
    assert np.array_equal(res.ids, want)
    assert res.rounds >= 3 and 1.0 < res.mean_tau < gamma + 1


def test_one_token_is_the_prefill_draw_and_no_round():
    """n_tokens = 1: the only token is the draw from the prefill's last logits
    (argmax when greedy, the inverse CDF at u_first when sampling); no round
    runs and the state holds the prompt alone."""
    cfg = es.tiny_c1()
    w = es.make_weights(cfg, seed=251)
    prompts = [es.prompt_tokens(cfg, L, seed=252 + b)[0] for b, L in enumerate((19, 7))]
    model = evs.Model(cfg, w, device=DEV)
    orc = HybridLM(cfg, w)
    from oracle.verifier import argmax_lowest, icdf, target_probs
    u_first = es.uniforms((2,), seed=255)
    for greedy in (True, False):
        state = evs.State(model, 2, 128, 8, device=DEV)
        res = evs.generate(model, state, prompts, 1, gamma=4, greedy=greedy, temperature=1.0, top_k=0,
                           table=np.zeros((2, 8), np.int32), u_first=u_first, u_target=es.uniforms((1, 2, 5), seed=256))
        assert res.rounds == 0 and res.ids.shape == (2, 1)
        for b, p in enumerate(prompts):
            lg, _ = orc.prefill(p, chunk=8)
            want = argmax_lowest(lg) if greedy else icdf(target_probs(lg, 1.0, 0), np.float32(u_first[b]),
                                                         argmax_lowest(lg))
            assert res.ids[b, 0] == want, (greedy, b)
        assert list(lengths(state)) == [len(p) for p in prompts]
        assert state.error() == 0
