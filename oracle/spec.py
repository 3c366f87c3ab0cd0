"""One speculative round, native decoding, and snapshot-and-replay.

A round (EvSpark preprint, abstract (i); Evo2 discussion #232, "What we
implemented"): the candidate block is [x_last, d_1 .. d_gamma], where x_last is
the last emitted token, not yet consumed. One block-verification forward gives
gamma+1 next-token distributions (row i predicts the token after candidate i,
so draft d_{i+1} is judged by row i). The verifier picks n_accepted; the state
is sliced to n_keep = n_accepted + 1 consumed positions; the emitted tokens are
d_1 .. d_{n_accepted} followed by the verifier's next token, which becomes the
new x_last.

``replay`` is the snapshot-and-replay scheme the pages contrast with
("The systems problem"): restore the pre-block snapshot and run the kept
tokens again one at a time. It defines what a correct rollback must equal.
"""
from __future__ import annotations

import numpy as np

from .verifier import verify_sample, verify_greedy, argmax_lowest


def spec_round(model, state, x_last, drafts, q=None, u=None, temperature=1.0,
               top_k=0, greedy=False):
    """Returns (n_accepted, next_token, new_state, pending)."""
    cand = np.concatenate([[int(x_last)], np.asarray(drafts, dtype=np.int64)])
    pend = model.block(state, cand)
    if greedy:
        n_acc, nxt = verify_greedy(pend.logits, drafts)
    else:
        n_acc, nxt = verify_sample(pend.logits, q, drafts, u, temperature, top_k)
    new_state = model.rollback(pend, n_acc + 1)
    return n_acc, nxt, new_state, pend


def native_greedy(model, state, x_last, n_tokens):
    """Greedy single-token decoding: consume x_last, emit argmax, repeat.
    Returns (tokens [n_tokens], final state)."""
    out = []
    s = state
    x = int(x_last)
    for _ in range(n_tokens):
        logits, s = model.step(s, x)
        x = argmax_lowest(logits)
        out.append(x)
    return np.asarray(out, dtype=np.int64), s


def replay(model, snapshot, tokens):
    """Snapshot-and-replay: consume ``tokens`` one at a time from ``snapshot``."""
    s = snapshot
    for t in tokens:
        _, s = model.step(s, int(t))
    return s
