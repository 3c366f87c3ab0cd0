"""Pins of oracle.spec.generate, the chained speculative rounds (model card,
"Library": generate equals generate_native token for token in greedy mode),
on the tiny fp32 stack: against step-by-step native decoding, greedy and
sampled, with the identity drafter, a corrupted (~75%) drafter and no drafter."""
import numpy as np

import evs_synth as es
from oracle import HybridLM
from oracle.spec import generate, native_greedy
from oracle.verifier import argmax_lowest, icdf, target_probs


def _model():
    cfg = es.tiny_c1()
    return cfg, HybridLM(cfg, es.make_weights(cfg, seed=7))


def _native_sampled(orc, prompt, n, u_first, u_steps, T, top_k):
    """Sequential single-token sampling: the definition."""
    s = orc.empty_state()
    for t in prompt:
        lg, s = orc.step(s, int(t))
    x = icdf(target_probs(lg, T, top_k), np.float32(u_first), argmax_lowest(lg))
    out = [x]
    for k in range(n - 1):
        lg, s = orc.step(s, x)
        x = icdf(target_probs(lg, T, top_k), np.float32(u_steps[k]), argmax_lowest(lg))
        out.append(x)
    return np.asarray(out)


def test_greedy_generation_equals_native_decoding_with_any_drafter():
    cfg, orc = _model()
    prompt = es.prompt_tokens(cfg, 24, seed=8)[0]
    n = 23
    _, st = orc.prefill(prompt, chunk=24)
    lg, _ = orc.prefill(prompt, chunk=24)
    first = argmax_lowest(lg)
    nat, _ = native_greedy(orc, st, first, n - 1)
    want = np.concatenate([[first], nat])
    ids0, r0, e0 = generate(orc, prompt, n, 0, greedy=True, prefill_chunk=24)
    assert np.array_equal(ids0, want) and r0 == n - 1 and e0 == n - 1
    table = np.concatenate([want, want[-1:].repeat(8)])
    for gamma in (1, 4, 6):
        ids, rounds, em = generate(orc, prompt, n, gamma, greedy=True, table=table, prefill_chunk=24)
        assert np.array_equal(ids, want), gamma
        assert rounds == -(-(n - 1) // (gamma + 1)), (gamma, rounds)      # every draft accepted
        # the ~75% drafter: a quarter of the slots replaced by another token
        rng = es.rng_for(9, "replace", gamma)
        rep = np.where(rng.random((n, gamma)) < 0.25, rng.integers(0, 4, (n, gamma)), -1)
        ids, rounds2, em2 = generate(orc, prompt, n, gamma, greedy=True, table=table, replace=rep, prefill_chunk=24)
        assert np.array_equal(ids, want), gamma
        assert rounds2 >= rounds and em2 >= n - 1


def test_sampled_generation_without_drafts_is_sequential_sampling():
    cfg, orc = _model()
    prompt = es.prompt_tokens(cfg, 16, seed=10)[0]
    n, T, top_k = 12, 0.8, 3
    u_first = es.uniforms((1,), seed=11)[0]
    u = es.uniforms((n, 1), seed=12)
    ids, rounds, _ = generate(orc, prompt, n, 0, temperature=T, top_k=top_k, u_first=u_first, u_target=u,
                              prefill_chunk=16)
    assert np.array_equal(ids, _native_sampled(orc, prompt, n, u_first, u[:, 0], T, top_k))
    assert rounds == n - 1


def test_truncation_at_n_tokens():
    cfg, orc = _model()
    prompt = es.prompt_tokens(cfg, 16, seed=13)[0]
    lg, _ = orc.prefill(prompt, chunk=16)
    ids, rounds, _ = generate(orc, prompt, 1, 4, greedy=True, table=np.zeros(8, np.int64), prefill_chunk=16)
    assert list(ids) == [argmax_lowest(lg)] and rounds == 0
    full, _, _ = generate(orc, prompt, 14, 0, greedy=True, prefill_chunk=16)
    table = np.concatenate([full, full[-1:].repeat(8)])
    for n in (2, 5, 6, 7, 14):
        ids, rounds, em = generate(orc, prompt, n, 5, greedy=True, table=table, prefill_chunk=16)
        assert np.array_equal(ids, full[:n]) and rounds == -(-(n - 1) // 6) and em == 6 * rounds, n


def tiny_drafter_f32(vocab=4, inject_dim=128):
    from evs_synth.configs import Block, ModelConfig
    return ModelConfig("tiny_drafter_f32", 64, vocab, [Block("attn", n_heads=2, head_dim=32), Block("mlp", d_ff=128)],
                       dtype="f32", inject_dim=inject_dim, max_slots=8)


def test_greedy_generation_with_a_drafter_model_equals_native():
    from oracle.drafter import Drafter
    cfg, orc = _model()
    dcfg = tiny_drafter_f32()
    dr = Drafter(dcfg, es.make_weights(dcfg, seed=14))
    prompt = es.prompt_tokens(cfg, 20, seed=15)[0]
    n = 17
    want, _, _ = generate(orc, prompt, n, 0, greedy=True, prefill_chunk=20)
    for gamma in (3, 8):
        ids, rounds, em = generate(orc, prompt, n, gamma, greedy=True, drafter=dr, export_block=1, prefill_chunk=20)
        assert np.array_equal(ids, want), gamma
        assert 1 <= rounds <= n - 1
