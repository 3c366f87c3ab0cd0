"""Drafter forward of the oracle (test infrastructure: only tests, the smoke
check and the benchmark's CPU baseline may import it).

What is computed (EvSpark preprint, abstract (ii): a distilled drafter made of
a gamma-parallel trunk, a prefix taken from the target's hidden state and a
full-matrix Markov head; model card, "Drafter checkpoints": one layer of
width 1024 injected from target layer 27, a frozen embedding, the Markov head,
and an exact causal prefix, so a checkpoint drafts any gamma' <= gamma).
The pages name these parts but give none of their formulas; the readings:

  * hidden-state export: h = the target's fp32 residual row after layer 27
    at the last consumed block position (the row whose logits produced the
    token the drafter continues from);
  * injection: z = st(st(rmsnorm(h)) W_inj^T), W_inj [d, inject_dim]. The RMS
    normalisation makes the prefix independent of the hidden state's scale
    (the pages report residual magnitudes near 1e11 in the last target blocks
    and carry them in fp32 for that reason);
  * slots: x_i = (E[x_last] + pos_i) + z for i = 0 .. gamma-1, with E the
    drafter's (frozen) token embedding and pos its position embeddings;
  * trunk: the drafter's blocks (one pre-norm causal attention + gated MLP
    layer) over the gamma slots from an empty state, then the final RMSNorm
    and the untied head: l_i = st(norm(x_i) W_o^T). Causal attention makes
    slot i independent of the slots after it (the exact causal prefix);
  * Markov head: l'_i = fp32(l_i) + T[d_{i-1}], T a full [V, V] fp32 matrix,
    d_{-1} = x_last, so the drafts are drawn one after another;
  * draft i: q_i = the verifier's target distribution of l'_i (temperature,
    top-k, the same fp32 sequential arithmetic); d_i = the inverse-CDF draw
    of q_i with the caller's uniform u_i (the argmax of l'_i if q_i has no
    positive entry), or the argmax of l'_i in greedy mode. The confidence head
    the checkpoints carry has no described use and is not computed.

Precision: the trunk as the hybrid oracle (fp64 with the model's storage
rounding); the Markov addition and the draws in fp32, because they decide
integers.

Parity pins (tests/test_oracle_drafter.py): the exact causal prefix (later
slots changed, earlier logits bit-identical), scale invariance of the
injection (h and 1e11 * h draft the same), and the Markov draws against the
closed form: with a zero head the drafts are a Markov chain whose transition
rows are the top-k softmax of T's rows (checked by exhaustive stratified
uniforms), and greedy drafts follow the argmax chain. Absolute values of the
random-init trunk logits have no printed reference (parity unpinned beyond
these invariants, as for the target stack).
"""
from __future__ import annotations

import numpy as np

from .hybrid import HybridLM
from .numerics import rmsnorm
from .verifier import argmax_lowest, icdf, target_probs

f32 = np.float32


class Drafter:
    """A drafter model: ``cfg`` is the drafter's config (inject_dim > 0) and
    ``weights`` its canonical tensors (the trunk's plus inject, pos, markov)."""

    def __init__(self, cfg, weights):
        if not cfg.inject_dim:
            raise ValueError("not a drafter config")
        self.cfg = cfg
        self.lm = HybridLM(cfg, weights)
        self.W = self.lm.W

    def prefix(self, hidden_row):
        """z = st(st(rmsnorm(h)) W_inj^T) for one exported target row h: the row
        is normalised before it is rounded to the storage type, so z does not
        depend on the row's overall scale."""
        h = np.asarray(hidden_row, dtype=np.float64)
        return self.lm.st(self.lm.st(rmsnorm(h, self.lm.eps)) @ self.W["inject"].T)

    def slots(self, hidden_row, last_tok: int, gamma: int):
        """Input rows of the gamma draft slots, [gamma, d]."""
        if not 0 < gamma <= self.cfg.max_slots:
            raise ValueError("gamma out of range")
        z = self.prefix(hidden_row)
        return (self.W["embed"][int(last_tok)][None, :] + self.W["pos"][:gamma]) + z[None, :]

    def trunk_logits(self, hidden_row, last_tok: int, gamma: int):
        """Head logits of the gamma slots (stored values), [gamma, V]."""
        X = self.slots(hidden_row, last_tok, gamma)
        return self.lm.block_rows(self.lm.empty_state(), X).logits

    def draft(self, logits, last_tok: int, u=None, temperature: float = 1.0, top_k: int = 0,
              greedy: bool = False):
        """Markov head and draws over the trunk logits [gamma, V]: returns
        (drafts [gamma] int32, q [gamma, V] fp32)."""
        logits = np.asarray(logits)
        gamma, V = logits.shape
        T = np.asarray(self.W["markov"], dtype=np.float32)
        drafts = np.zeros(gamma, dtype=np.int32)
        q = np.zeros((gamma, V), dtype=np.float32)
        prev = int(last_tok)
        for i in range(gamma):
            lp = (np.asarray(logits[i], dtype=np.float32) + T[prev]).astype(np.float32)
            q[i] = target_probs(lp, temperature, top_k)
            if greedy:
                d = argmax_lowest(lp)
            else:
                d = icdf(q[i], f32(u[i]), argmax_lowest(lp))
            drafts[i] = d
            prev = d
        return drafts, q

    def forward(self, hidden_row, last_tok: int, gamma: int, u=None, temperature: float = 1.0,
                top_k: int = 0, greedy: bool = False):
        """Trunk logits, then the drafts: (drafts, q, logits)."""
        lg = self.trunk_logits(hidden_row, last_tok, gamma)
        d, q = self.draft(lg, last_tok, u, temperature, top_k, greedy)
        return d, q, lg
