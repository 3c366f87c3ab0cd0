"""Pins of the oracle's verifier.

The central pin is the theorem the pages state (EvSpark preprint, abstract
(iii)): in exact arithmetic, speculative sampling with rejection-sampling
verification emits tokens distributed exactly as the target model. It is
checked by exhaustive enumeration: every draft sequence (weighted by the
drafter's probabilities) and a stratified grid of uniforms, on distributions
whose entries are multiples of 1/8 with drafter entries that are powers of two
and residual masses in {0, 1/8, 1/4, 1/2}. On such inputs every threshold the
verifier compares against lies on a grid-cell boundary and every fp32
operation is exact, so the grid average IS the exact output probability and is
compared with the target's autoregressive probability as rational numbers.
"""
import itertools
from collections import defaultdict
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax

from oracle.verifier import (argmax_lowest, icdf, target_probs, verify_greedy,
                             verify_sample)

V = 4
G_ACC, G_FIN = 4, 8


class DyadicTables:
    """Prefix-indexed target p(.|prefix) and drafter q(.|prefix) tables."""

    def __init__(self, seed):
        self.seed = seed
        self.cache = {}

    def rows(self, prefix):
        key = tuple(prefix)
        if key not in self.cache:
            rng = np.random.default_rng([self.seed] + [t + 1 for t in key] + [99])
            q8 = list(rng.permutation([4, 2, 1, 1]))
            while True:
                s_units = int(rng.choice([0, 1, 2, 4]))
                removed = [0] * V
                for _ in range(s_units):
                    cand = [i for i in range(V) if q8[i] - removed[i] > 0]
                    removed[int(rng.choice(cand))] += 1
                A = {i for i in range(V) if removed[i]}
                B = [i for i in range(V) if i not in A]
                if s_units and not B:
                    continue
                added = [0] * V
                for _ in range(s_units):
                    added[int(rng.choice(B))] += 1
                break
            p8 = [q8[i] - removed[i] + added[i] for i in range(V)]
            self.cache[key] = (np.array(p8, np.float32) / 8, np.array(q8, np.float32) / 8,
                               [Fraction(x, 8) for x in p8], [Fraction(x, 8) for x in q8])
        return self.cache[key]


def round_outcomes(tab, prefix, gamma):
    out = defaultdict(Fraction)
    grid_acc = [(j + 0.5) / G_ACC for j in range(G_ACC)]
    grid_fin = [(j + 0.5) / G_FIN for j in range(G_FIN)]
    cell = Fraction(1, G_ACC ** gamma * G_FIN)
    for drafts in itertools.product(range(V), repeat=gamma):
        w = Fraction(1)
        for i in range(gamma):
            w *= tab.rows(prefix + drafts[:i])[3][drafts[i]]
        if w == 0:
            continue
        target = np.stack([tab.rows(prefix + drafts[:i])[0] for i in range(gamma + 1)])
        qrows = np.stack([tab.rows(prefix + drafts[:i])[1] for i in range(gamma)])
        for ua in itertools.product(grid_acc, repeat=gamma):
            for uf in grid_fin:
                u = np.array(list(ua) + [uf], np.float32)
                n_acc, nxt = verify_sample(target, qrows, np.array(drafts), u, target_is_probs=True)
                out[tuple(drafts[:n_acc]) + (nxt,)] += w * cell
    return out


def emitted_distribution(tab, prefix, gamma, m, memo):
    key = (prefix, m)
    if key in memo:
        return memo[key]
    res = defaultdict(Fraction)
    for emitted, pr in round_outcomes(tab, prefix, gamma).items():
        if len(emitted) >= m:
            res[emitted[:m]] += pr
        else:
            for rest, pr2 in emitted_distribution(tab, prefix + emitted, gamma, m - len(emitted), memo).items():
                res[emitted + rest] += pr * pr2
    memo[key] = res
    return res


@pytest.mark.parametrize("gamma,m,seed", [(1, 3, 0), (2, 3, 1), (2, 2, 2), (3, 1, 3)])
def test_rejection_sampler_preserves_target_distribution_exactly(gamma, m, seed):
    tab = DyadicTables(seed)
    got = emitted_distribution(tab, (), gamma, m, {})
    for seq in itertools.product(range(V), repeat=m):
        want = Fraction(1)
        for j in range(m):
            want *= tab.rows(seq[:j])[2][seq[j]]
        assert got.get(seq, Fraction(0)) == want, (seq, got.get(seq), want)
    assert sum(got.values()) == 1


def test_plausible_verifier_mistake_would_be_caught():
    """Sanity of the pin itself: a residual taken as max(0, q - p) breaks it."""
    tab = DyadicTables(1)
    p, q = tab.rows(())[0], tab.rows(())[1]
    if np.array_equal(p, q):
        pytest.skip("degenerate table row")
    # exact output distribution of the first token with the correct verifier
    got = emitted_distribution(tab, (), 1, 1, {})
    want = tab.rows(())[2]
    assert [got.get((y,), 0) for y in range(V)] == want
    wrong_resid = np.maximum(0, q - p)
    assert not np.allclose(wrong_resid / max(wrong_resid.sum(), 1e-9),
                           np.maximum(0, p - q) / max(np.maximum(0, p - q).sum(), 1e-9))


def test_accept_and_residual_worked_case():
    p = np.array([[0.5, 0.5, 0, 0], [0, 0, 1.0, 0]], np.float32)
    q = np.array([[1.0, 0, 0, 0]], np.float32)
    # u0 = 0.4 < p/q = 0.5: accept, bonus from row 1 -> token 2
    assert verify_sample(p, q, [0], np.array([0.4, 0.3], np.float32), target_is_probs=True) == (1, 2)
    # u0 = 0.6: reject; residual max(0, p - q) = [0, .5, 0, 0] -> token 1
    assert verify_sample(p, q, [0], np.array([0.6, 0.99], np.float32), target_is_probs=True) == (0, 1)
    # draft with q = 0 and p > 0 is accepted
    q2 = np.array([[0.0, 1.0, 0, 0]], np.float32)
    assert verify_sample(p, q2, [0], np.array([0.99, 0.5], np.float32), target_is_probs=True)[0] == 1


def test_icdf_rules():
    w = np.array([0.0, 0.25, 0.0, 0.75], np.float32)
    assert icdf(w, 0.0, 9) == 1
    assert icdf(w, 0.2499, 9) == 1
    assert icdf(w, 0.25, 9) == 3            # strict '>' on the running sum
    assert icdf(w, 1.5, 9) == 3             # past the end: last positive entry
    assert icdf(np.zeros(4, np.float32), 0.1, 9) == 9


def test_target_probs_softmax_and_topk():
    rng = np.random.default_rng(0)
    z = rng.standard_normal(64).astype(np.float32)
    p = target_probs(z, 1.0, 0)
    assert np.allclose(p, softmax(z.astype(np.float64)), rtol=1e-6, atol=1e-9)
    pt = target_probs(z, 0.7, 0)
    assert np.allclose(pt, softmax(z.astype(np.float64) / np.float32(0.7)), rtol=1e-5, atol=1e-9)
    # top-k keeps the k largest; ties at the cut go to the lower id
    zt = np.array([1.0, 3.0, 2.0, 3.0, 2.0, 0.0], np.float32)
    p2 = target_probs(zt, 1.0, 3)
    assert list(np.nonzero(p2)[0]) == [1, 2, 3]
    assert np.allclose(p2[[1, 2, 3]], softmax(np.array([3.0, 2.0, 3.0])), rtol=1e-6)
    # NaN logits never survive; a row of NaN has no mass
    zn = zt.copy()
    zn[1] = np.nan
    assert target_probs(zn, 1.0, 0)[1] == 0
    assert not target_probs(np.full(4, np.nan, np.float32), 1.0, 0).any()


def test_greedy_rules():
    logits = np.array([[0.0, 2.0, 2.0, 1.0],     # tie: lowest id (1) wins
                       [5.0, 0.0, 0.0, 0.0],
                       [0.0, 0.0, 0.0, 7.0]], np.float32)
    assert argmax_lowest(logits[0]) == 1
    assert verify_greedy(logits, [1, 0]) == (2, 3)       # all accepted, bonus argmax
    assert verify_greedy(logits, [2, 0]) == (0, 1)       # mismatch at 0 emits argmax
    assert verify_greedy(logits, [1, 3]) == (1, 0)
    assert argmax_lowest(np.array([np.nan, 1.0, np.nan], np.float32)) == 1
    # NaN reads as -inf in a logits row but as probability 0 in a probability
    # row: [NaN, 0, 0] has its maximum at id 1 as logits and at id 0 (every
    # entry 0, lowest id) as probabilities
    nanrow = np.array([[np.nan, 0.0, 0.0]], np.float32)
    assert verify_greedy(nanrow, []) == (0, 1)
    assert verify_greedy(nanrow, [], target_is_probs=True) == (0, 0)


def test_degenerate_target_falls_back_to_argmax():
    """A logits row with no finite entry gives p = 0 everywhere: the draft is
    rejected and the draw falls back to the row's argmax (token 0 for all-NaN)."""
    t = np.array([[np.nan] * 4, [0.0, 1.0, 0.0, 0.0]], np.float32)
    q = np.array([[0.25] * 4], np.float32)
    assert verify_sample(t, q, [2], np.array([0.1, 0.5], np.float32)) == (0, 0)
