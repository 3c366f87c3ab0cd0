"""One speculative round, native decoding, and snapshot-and-replay.

Part of the oracle: test infrastructure only (the tests, the smoke check and
the benchmark's CPU-baseline leg may import it; the HIP path never does).

A round (EvSpark preprint, abstract (i); Evo2 discussion #232, "What we
implemented"): the candidate block is [x_last, d_1 .. d_gamma], where x_last is
the last emitted token, not yet consumed. One block-verification forward gives
gamma+1 next-token distributions (row i predicts the token after candidate i,
so draft d_{i+1} is judged by row i). The verifier picks n_accepted; the state
is sliced to n_keep = n_accepted + 1 consumed positions; the emitted tokens are
d_1 .. d_{n_accepted} followed by the verifier's next token, which becomes the
new x_last.

``generate`` chains rounds into the generation loop of the library the
model card describes (generate / generate_native), truncated at n_tokens.

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


def generate(model, prompt, n_tokens, gamma, greedy=False, temperature=1.0, top_k=0, u_first=None,
             u_target=None, drafter=None, export_block=None, u_draft=None, table=None, replace=None,
             prefill_chunk=256):
    """Generation by chained speculative rounds for one sequence (model card,
    "Library": generate, and generate_native with gamma = 0).

    The prompt is consumed (prefill); the first new token is drawn from the
    last prompt position's logits (the argmax when greedy, else the inverse
    CDF of the target distribution at u_first). Then each round r drafts
    gamma tokens after the last emitted token x_last and verifies them
    (``spec_round`` with u_target[r]); with gamma = 0 a round is one native
    step. The drafts come from
      * ``drafter`` (an oracle.drafter.Drafter): its forward over the target's
        residual row after block ``export_block`` at the last consumed
        position, with u_draft[r];
      * ``table``: the proposal for generated token k is table[k] (clamped to
        the table's end), so after e emitted tokens draft i is
        table[e + i - 1]; where replace[r][i] >= 0 the slot takes that token
        instead; q is one-hot at each draft.
    A round emits d_1 .. d_{n_acc} and the verifier's next token. Generation
    stops at n_tokens: if a round would pass it, only the first r = n_tokens
    - emitted of its tokens are emitted and only r positions are kept.
    Returns (ids [n_tokens], rounds, tokens emitted by the rounds before any
    truncation), so tokens per round = that count / rounds."""
    from .verifier import icdf, target_probs
    prompt = np.asarray(prompt)
    state = model.empty_state()
    hidden = None
    for a in range(0, len(prompt), prefill_chunk):
        pend = model.block(state, prompt[a:a + prefill_chunk], keep_x=drafter is not None)
        state = model.rollback(pend, pend.P)
        last_logits = pend.logits[-1]
        if drafter is not None:
            hidden = pend.x_out[export_block][-1]
    if greedy:
        x = argmax_lowest(last_logits)
    else:
        p = target_probs(last_logits, temperature, top_k)
        x = icdf(p, np.float32(u_first), argmax_lowest(last_logits))
    ids = [int(x)]
    rounds = emitted_untrunc = 0
    while len(ids) < n_tokens:
        r = rounds
        q = None
        if gamma == 0:
            drafts = np.zeros(0, dtype=np.int64)
        elif drafter is not None:
            drafts, q, _ = drafter.forward(hidden, x, gamma, None if greedy else u_draft[r], temperature, top_k, greedy)
        else:
            e = len(ids)
            drafts = np.array([table[min(e + i - 1, len(table) - 1)] for i in range(1, gamma + 1)], dtype=np.int64)
            if replace is not None:
                drafts = np.where(np.asarray(replace[r]) >= 0, replace[r], drafts)
            q = np.zeros((gamma, len(last_logits)), dtype=np.float32)
            q[np.arange(gamma), drafts] = 1.0
        cand = np.concatenate([[int(x)], np.asarray(drafts, dtype=np.int64)])
        pend = model.block(state, cand, keep_x=drafter is not None)
        if greedy:
            n_acc, nxt = verify_greedy(pend.logits, drafts)
        else:
            n_acc, nxt = verify_sample(pend.logits, q, drafts, u_target[r], temperature, top_k)
        out = [int(t) for t in drafts[:n_acc]] + [int(nxt)]
        rounds += 1
        emitted_untrunc += len(out)
        take = min(len(out), n_tokens - len(ids))
        ids += out[:take]
        state = model.rollback(pend, take)        # positions x_last, d_1 .. d_{take-1}
        x = ids[-1]
        if drafter is not None:
            hidden = pend.x_out[export_block][take - 1]
    return np.asarray(ids, dtype=np.int64), rounds, emitted_untrunc
