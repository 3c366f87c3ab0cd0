"""Pins of the oracle drafter (oracle/drafter.py) against properties the pages
fix and closed forms: the exact causal prefix, the scale invariance of the
hidden-state injection, and the Markov head's draws."""
import itertools

import numpy as np
import torch

import evs_synth as es
from evs_synth.configs import Block, ModelConfig
from oracle.drafter import Drafter


def tiny_drafter(vocab=16):
    return ModelConfig("tiny_drafter", 128, vocab, [Block("attn", n_heads=4, head_dim=32), Block("mlp", d_ff=352)],
                       dtype="bf16", inject_dim=96, max_slots=8)


def hidden(seed, n=96, scale=1.0):
    return es.rng_for(seed, "hidden").standard_normal(n) * scale


def test_exact_causal_prefix():
    """Changing a later slot leaves every earlier slot's logits bit-identical
    (same shapes, so the same arithmetic per row); a shorter gamma drafts the
    same leading tokens (model card: any gamma' <= gamma is an exact prefix)."""
    cfg = tiny_drafter()
    w = es.make_weights(cfg, seed=1)
    dr = Drafter(cfg, w)
    h = hidden(2)
    base = dr.trunk_logits(h, 3, 6)
    w2 = dict(w)
    pos = w["pos"].clone()
    pos[5] = pos[5] * 50 + 1
    w2["pos"] = pos
    other = Drafter(cfg, w2).trunk_logits(h, 3, 6)
    assert np.array_equal(base[:5], other[:5])
    assert not np.array_equal(base[5], other[5])
    short = dr.trunk_logits(h, 3, 4)
    assert np.max(np.abs(short - base[:4])) <= 2.0 ** -7 * np.max(np.abs(base[:4]))
    u = es.uniforms((6,), seed=3)
    d6, _ = dr.draft(base, 3, u)
    d4, _ = dr.draft(base[:4], 3, u[:4])
    assert np.array_equal(d6[:4], d4)


def test_injection_is_scale_invariant():
    """The prefix is RMS-normalised: a hidden row scaled by 1e11 (the
    magnitude the pages report for the last target blocks) drafts as the
    unscaled row; a different row changes the logits."""
    cfg = tiny_drafter()
    dr = Drafter(cfg, es.make_weights(cfg, seed=4))
    h = hidden(5)
    a = dr.trunk_logits(h, 1, 5)
    b = dr.trunk_logits(h * 1e11, 1, 5)
    assert np.max(np.abs(a - b)) <= 2e-2
    assert np.mean(a == b) > 0.95
    c = dr.trunk_logits(hidden(6), 1, 5)
    assert np.max(np.abs(a - c)) > 1e-3
    assert np.array_equal(dr.prefix(h * 1e11), dr.prefix(h)) or np.max(np.abs(dr.prefix(h * 1e11) - dr.prefix(h))) < 1e-2


def _zero_head(vocab, seed):
    cfg = tiny_drafter(vocab)
    w = es.make_weights(cfg, seed=seed)
    w["lm_head"] = torch.zeros_like(w["lm_head"])
    return cfg, w


def _closed_form_rows(T, temperature, top_k):
    T = np.asarray(T, np.float64) / temperature
    V = T.shape[1]
    out = np.zeros_like(T)
    for x in range(T.shape[0]):
        keep = np.argsort(-T[x], kind="stable")[: (top_k if 0 < top_k < V else V)]
        e = np.exp(T[x, keep] - T[x, keep].max())
        out[x, keep] = e / e.sum()
    return out


def test_markov_draws_match_the_transition_closed_form():
    """With a zero head the trunk logits are exactly 0, so the drafts form a
    Markov chain whose rows are the top-k softmax of T / temperature. Over a
    stratified grid of uniforms for two positions, the joint frequency of every
    (d_0, d_1) equals p(d_0 | x_last) p(d_1 | d_0) within the grid's
    resolution."""
    V, G = 4, 256
    cfg, w = _zero_head(V, 7)
    dr = Drafter(cfg, w)
    lg = dr.trunk_logits(hidden(8), 2, 2)
    assert np.all(lg == 0)
    for temperature, top_k in ((1.0, 0), (0.6, 3)):
        p = _closed_form_rows(w["markov"].numpy(), temperature, top_k)
        grid = (np.arange(G) + 0.5) / G
        freq = np.zeros((V, V))
        for u0, u1 in itertools.product(grid, grid):
            d, q = dr.draft(lg, 2, np.array([u0, u1], np.float32), temperature, top_k)
            freq[d[0], d[1]] += 1.0 / G ** 2
        expect = p[2][:, None] * p
        assert np.max(np.abs(freq - expect)) <= 2.0 / G, (temperature, top_k)
        # q of each position is that position's transition row
        d, q = dr.draft(lg, 2, np.array([0.3, 0.7], np.float32), temperature, top_k)
        assert np.allclose(q[0], p[2], atol=1e-6) and np.allclose(q[1], p[d[0]], atol=1e-6)


def test_greedy_drafts_follow_the_argmax_chain():
    V = 16
    cfg, w = _zero_head(V, 9)
    dr = Drafter(cfg, w)
    lg = dr.trunk_logits(hidden(10), 5, 7)
    d, _ = dr.draft(lg, 5, greedy=True)
    T = w["markov"].numpy()
    prev, chain = 5, []
    for _ in range(7):
        prev = int(np.argmax(T[prev]))
        chain.append(prev)
    assert list(d) == chain
