"""Verification of a drafted block: exact rejection sampling and greedy.

Part of the oracle: test infrastructure only (the tests, the smoke check and
the benchmark's CPU-baseline leg may import it; the HIP path never does).

Sampling mode follows the exact rejection-sampling verifier the pages name
(EvSpark preprint, abstract (iii): the scheme preserves the target
distribution in exact arithmetic; Evo2 discussion #232, "A few other
observations": exact rejection-sampling verification rather than an
approximate acceptance rule). Its steps, for one sequence with drafts
d_1..d_gamma, draft distributions q_i, target distributions p_0..p_gamma and
uniforms u_0..u_gamma:

  1. target p_i = softmax over the top_k largest of logits_i / T (ties in the
     top-k cut go to the lower token id; top_k of 0 or >= V keeps all);
  2. for i = 0 .. gamma-1 with x = d_{i+1}: accept if u_i < p_i[x] / q_i[x]
     (when q_i[x] > 0; else accept iff p_i[x] > 0); stop at the first reject;
  3. at a reject at i: draw the next token from the residual
     max(0, p_i - q_i) normalised (from p_i if the residual is all zero);
  4. if all gamma drafts are accepted: draw a bonus token from p_gamma;
  5. a draw from weights w with uniform u is the inverse CDF: the first token
     y whose running sum of w exceeds u * sum(w) (the last token with
     positive weight if rounding leaves none).

Greedy mode (model card, "Library": greedy output equals native decoding token
for token): accept d_{i+1} iff it is the argmax of logits_i (lowest id among
equal maxima); at the first mismatch emit that argmax; if all are accepted emit
the argmax of logits_gamma.

Precision: every step runs in fp32, the precision the GPU decides in, because
these floating-point values decide integers. Sums run sequentially in
increasing token order; exp is evaluated in fp64 and rounded to fp32; NaN
logits count as -inf and NaN probabilities as 0; if a target row has no
positive entry the draw falls back to the argmax of its logits (of its
probabilities in probability mode, token 0 if all are NaN).

Parity pins (tests/test_oracle_verifier.py): the output distribution of chained
rounds equals the target's autoregressive distribution exactly, by enumeration
over drafts and a stratified uniform grid on dyadic distributions; greedy rules
and the identity drafter; top-k tie order; degenerate rows.
"""
from __future__ import annotations

import numpy as np

f32 = np.float32


def _clean_logits(row):
    z = np.asarray(row, dtype=np.float32).copy()
    z[np.isnan(z)] = -np.inf
    return z


def argmax_lowest(row) -> int:
    """Index of the maximum, lowest index among ties; NaN counts as -inf."""
    z = _clean_logits(row)
    best, arg = -np.inf, 0
    for y in range(len(z)):
        if z[y] > best:
            best, arg = z[y], y
    return arg


def target_probs(logits_row, temperature: float = 1.0, top_k: int = 0) -> np.ndarray:
    """fp32 target distribution from one row of logits (step 1)."""
    z = _clean_logits(logits_row) / f32(temperature)
    V = len(z)
    keep = np.zeros(V, dtype=bool)
    if top_k <= 0 or top_k >= V:
        keep[:] = True
    else:
        order = sorted(range(V), key=lambda y: (-float(z[y]), y))
        keep[order[:top_k]] = True
    keep &= np.isfinite(z)
    if not keep.any():
        return np.zeros(V, dtype=np.float32)
    m = z[keep].max()
    e = np.zeros(V, dtype=np.float32)
    for y in range(V):
        if keep[y]:
            e[y] = f32(np.exp(np.float64(f32(z[y] - m))))
    S = f32(0.0)
    for y in range(V):
        S = f32(S + e[y])
    p = np.zeros(V, dtype=np.float32)
    for y in range(V):
        p[y] = f32(e[y] / S)
    return p


def icdf(w, u, fallback: int) -> int:
    """Inverse-CDF draw (step 5): first y with running fp32 sum of w > u."""
    c = f32(0.0)
    u = f32(u)
    last_pos = -1
    for y in range(len(w)):
        c = f32(c + w[y])
        if w[y] > 0:
            last_pos = y
        if c > u:
            return y
    return last_pos if last_pos >= 0 else fallback


def _clean_probs(row):
    p = np.asarray(row, dtype=np.float32).copy()
    p[np.isnan(p)] = 0
    return p


def verify_sample(target, q, drafts, u, temperature=1.0, top_k=0, target_is_probs=False):
    """Rejection-sampling verification of one sequence.

    target: [gamma+1, V] logits (or probabilities if ``target_is_probs``);
    q: [gamma, V] draft distributions; drafts: [gamma] token ids;
    u: [gamma+1] fp32 uniforms (u[i] for the accept test of draft i+1, u[gamma]
    for the final draw). Returns (n_accepted, next_token).
    """
    target = np.asarray(target)
    gamma = len(drafts)
    V = target.shape[-1]
    if target_is_probs:
        P = [_clean_probs(target[i]) for i in range(gamma + 1)]
    else:
        P = [target_probs(target[i], temperature, top_k) for i in range(gamma + 1)]

    def fallback(i):
        return argmax_lowest(P[i] if target_is_probs else target[i])

    uf = np.asarray(u, dtype=np.float32)
    for i in range(gamma):
        x = int(drafts[i])
        if not 0 <= x < V:
            raise ValueError("draft token out of range")
        px = P[i][x]
        qi = _clean_probs(q[i])
        qx = qi[x]
        if qx > 0:
            ok = uf[i] < f32(px / qx)
        else:
            ok = px > 0
        if not ok:
            w = np.zeros(V, dtype=np.float32)
            for y in range(V):
                w[y] = max(f32(0.0), f32(P[i][y] - qi[y]))
            S = f32(0.0)
            for y in range(V):
                S = f32(S + w[y])
            if S > 0:
                nxt = icdf(w, f32(uf[gamma] * S), fallback(i))
            else:
                nxt = icdf(P[i], uf[gamma], fallback(i))
            return i, nxt
    return gamma, icdf(P[gamma], uf[gamma], fallback(gamma))


def verify_greedy(target, drafts, target_is_probs=False):
    """Greedy verification of one sequence: (n_accepted, next_token). With
    probability targets a NaN entry reads as probability 0 (as in sampling
    mode); with logits it reads as -inf."""
    gamma = len(drafts)
    rows = [_clean_probs(target[i]) if target_is_probs else target[i] for i in range(gamma + 1)]
    for i in range(gamma):
        a = argmax_lowest(rows[i])
        if int(drafts[i]) != a:
            return i, a
    return gamma, argmax_lowest(rows[gamma])
