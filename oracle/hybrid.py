"""The hybrid (FIR / IIR / attention + MLP) stack, in two independent forms.

Part of the oracle: test infrastructure only (the tests, the smoke check and
the benchmark's CPU-baseline leg may import it; the HIP path never does).

What is computed (EvSpark preprint, abstract (i); Evo2 discussion #232, "The
systems problem" and "What we implemented"): a StripedHyena2-style stack whose
inference state mixes three classes — fixed-length FIR sliding windows, IIR
recurrent states that depend on the whole accepted prefix, and append-only
attention KV caches. The pages give no layer formulas; the readings used here:

  * model   = embedding -> pre-norm residual blocks -> RMSNorm -> untied LM head;
  * norm    = RMSNorm, unit gain, eps from the config, feeding a product:
              norm(x) W^T = r * (x W^T) with r = 1 / sqrt(mean(x^2) + eps);
              the product's operand is the residual row rounded to the
              storage type and r scales the product's sum (the mixer, the MLP
              and the LM head alike);
  * mixer   = z = u W_in^T split [q | k | v]; h = k * v; y = op(h); o = q * y;
              x += o W_out^T, where op is
      FIR   : y_t[c] = sum_{j<L} taps[c, j] * h_{t-j}[c]   (h before position 0 is 0);
              state = the last L-1 inputs h (the sliding window);
      IIR   : s_t[c, n] = lam[c, n] * s_{t-1}[c, n] + h_t[c], s_{-1} = 0;
              y_t[c] = sum_n res[c, n] * s_t[c, n]; state = s;
      ATTN  : causal multi-head softmax(q k^T / sqrt(Dh)) v, no positional
              encoding; state = the K and V rows (append-only);
  * MLP     = x += (gelu(u W_g^T) * (u W_u^T)) W_down^T, gate rows first in W_gu;
  * storage = projection outputs, mixer outputs, KV rows, MLP hidden and logits
              are rounded to the storage type (bf16 models); the residual
              stream and the FIR/IIR states are kept unrounded.

Step form (``step``): one token at a time — sequential single-token decoding,
the definition of the result (model card, "Library": greedy speculative output
equals native decoding token for token).

Block form (``block``): the block-verification forward over P = gamma+1
candidate tokens in one pass, keeping the state of every position
("What we implemented": the intermediate state of each position in the
speculative block is retained), written with batched matrix products, a
slice-sum convolution and a masked attention matrix. ``rollback`` slices the
per-position state to the accepted boundary with no recomputation.

Parity pins (tests/test_oracle_model.py): FIR op against scipy.signal.lfilter;
IIR op against its impulse-response convolution; attention against closed
forms; block form against step form; rollback against replay; a hand-worked
two-channel stack; causal-prefix and identity-drafter invariants. Absolute
values of random-init logits have no printed reference ("parity unpinned"
beyond these invariants).
"""
from __future__ import annotations

import copy
from dataclasses import dataclass, field
from typing import Dict

import numpy as np

from .numerics import gelu, rms_scale, store


def _f64(t):
    if hasattr(t, "detach"):
        t = t.detach().to("cpu").float().numpy()
    return np.asarray(t, dtype=np.float64)


@dataclass
class SeqState:
    """Committed inference state of one sequence after ``t`` consumed tokens."""
    t: int = 0
    fir: Dict[int, np.ndarray] = field(default_factory=dict)  # [L-1, d]: h at t-L+1 .. t-1
    iir: Dict[int, np.ndarray] = field(default_factory=dict)  # [d, N]
    k: Dict[int, np.ndarray] = field(default_factory=dict)    # [t, H, Dh]
    v: Dict[int, np.ndarray] = field(default_factory=dict)    # [t, H, Dh]

    def clone(self) -> "SeqState":
        return copy.deepcopy(self)


@dataclass
class Pending:
    """Result of a block-verify forward: logits of every candidate position and
    the per-position state, not yet committed."""
    base: SeqState
    tokens: np.ndarray
    logits: np.ndarray                                          # [P, V]
    fir_h: Dict[int, np.ndarray] = field(default_factory=dict)  # [P, d]
    iir_s: Dict[int, np.ndarray] = field(default_factory=dict)  # [P, d, N]
    k_new: Dict[int, np.ndarray] = field(default_factory=dict)  # [P, H, Dh]
    v_new: Dict[int, np.ndarray] = field(default_factory=dict)  # [P, H, Dh]
    x_out: Dict[int, np.ndarray] = field(default_factory=dict)  # residual after block i, [P, d]
    z: Dict[int, np.ndarray] = field(default_factory=dict)      # mixer in-projection [q|k|v], [P, 3d]

    @property
    def P(self):
        return len(self.tokens)

    def fir_window(self, i: int, p: int) -> np.ndarray:
        """FIR state of block i after candidate position p: the last L-1 inputs."""
        full = np.vstack([self.base.fir[i], self.fir_h[i][: p + 1]])
        return full[-self.base.fir[i].shape[0]:] if self.base.fir[i].shape[0] else full[:0]


def fir_conv(hist, Hh, taps):
    """Causal depthwise FIR over a block: hist [L-1, d] holds the inputs at the
    L-1 positions before the block (oldest first), Hh [P, d] the block's inputs,
    taps [d, L] with tap j applied to the input j steps back. Returns Y [P, d]."""
    L, P = taps.shape[1], Hh.shape[0]
    seq = np.vstack([hist, Hh])                   # positions t-L+1 .. t+P-1
    Y = np.zeros(Hh.shape)
    for j in range(L):
        Y += taps[:, j][None, :] * seq[L - 1 - j: L - 1 - j + P]
    return Y


def iir_scan(s0, Hh, lam, res):
    """Diagonal modal recurrence over a block from state s0 [d, N]:
    s_p = lam * s_{p-1} + h_p (broadcast over modes), y_p = sum_n res * s_p.
    Returns (Y [P, d], S [P, d, N] — the state after every position)."""
    P = Hh.shape[0]
    S = np.zeros((P,) + s0.shape)
    s = s0
    for p in range(P):
        s = lam * s + Hh[p][:, None]
        S[p] = s
    return np.einsum("cn,pcn->pc", res, S), S


def causal_attention(Kc, Vc, Qh, Kn, Vn):
    """Block-causal multi-head attention: the cache holds t rows (Kc, Vc
    [t, H, Dh]); the block appends P rows (Kn, Vn) and query p (position t+p)
    attends to keys 0 .. t+p with softmax(q k / sqrt(Dh)). Returns [P, H, Dh]."""
    t, P, Dh = Kc.shape[0], Qh.shape[0], Qh.shape[2]
    Ka = np.concatenate([Kc, Kn], axis=0)         # [t+P, H, Dh]
    Va = np.concatenate([Vc, Vn], axis=0)
    scores = np.einsum("phd,jhd->hpj", Qh, Ka) / np.sqrt(Dh)
    visible = np.arange(t + P)[None, :] <= (t + np.arange(P))[:, None]
    scores = np.where(visible[None], scores, -np.inf)
    w = np.exp(scores - scores.max(axis=-1, keepdims=True))
    w /= w.sum(axis=-1, keepdims=True)
    return np.einsum("hpj,jhd->phd", w, Va)


class HybridLM:
    def __init__(self, cfg, weights, accumulate: str = "f64"):
        """accumulate: "f64" (the reference: every product and sum of a
        matrix product in float64) or "f32" (the block form's matrix products
        accumulate in float32, as an implementation with fp32 accumulators
        does; operands are the same stored values, so only the rounding of
        the sums differs). The step form always uses float64."""
        if accumulate not in ("f64", "f32"):
            raise ValueError(accumulate)
        self.cfg = cfg
        self.d = cfg.d_model
        self.W = {k: _f64(v) for k, v in weights.items()}
        self.dt = cfg.dtype
        self.eps = float(cfg.norm_eps)
        self.acc = accumulate

    def st(self, x):
        return store(x, self.dt)

    def mm(self, A, W):
        """A @ W^T with the block form's accumulation (see __init__)."""
        if self.acc == "f32":
            return (np.asarray(A, np.float32) @ np.asarray(W, np.float32).T).astype(np.float64)
        return A @ W.T

    def with_accumulation(self, accumulate: str) -> "HybridLM":
        """The same model (weights shared, not copied) with another accumulation."""
        if accumulate not in ("f64", "f32"):
            raise ValueError(accumulate)
        other = copy.copy(self)
        other.acc = accumulate
        return other

    def normed_mm(self, X, W):
        """norm(X) W^T for residual rows X [P, d]: the rows rounded to the
        storage type as the operand, each row's RMSNorm scale on the sum."""
        X = np.asarray(X, dtype=np.float64)
        return rms_scale(X, self.eps) * self.mm(self.st(X), W)

    def head(self, X):
        """Logits of residual rows X [P, d]: final RMSNorm and the LM head."""
        return self.st(self.normed_mm(X, self.W["lm_head"]))

    # ------------------------------------------------------------------ state
    def empty_state(self) -> SeqState:
        s = SeqState(t=0)
        for i, b in enumerate(self.cfg.blocks):
            if b.kind == "fir":
                s.fir[i] = np.zeros((b.fir_len - 1, self.d))
            elif b.kind == "iir":
                s.iir[i] = np.zeros((self.d, b.iir_states))
            elif b.kind == "attn":
                s.k[i] = np.zeros((0, b.n_heads, b.head_dim))
                s.v[i] = np.zeros((0, b.n_heads, b.head_dim))
        return s

    def import_state(self, t: int, synth) -> SeqState:
        """Committed state from ``evs_synth.synthetic_state`` output."""
        s = SeqState(t=t)
        for i, b in enumerate(self.cfg.blocks):
            if b.kind == "fir":
                s.fir[i] = _f64(synth[i]["hist"])
            elif b.kind == "iir":
                s.iir[i] = _f64(synth[i]["s"])
            elif b.kind == "attn":
                s.k[i] = _f64(synth[i]["k"])
                s.v[i] = _f64(synth[i]["v"])
        return s

    # ------------------------------------------------------- step form (definition)
    def step(self, state: SeqState, token: int):
        """Consume one token: returns (logits [V], new state). The input state is
        not modified."""
        s = state.clone()
        x = self.W["embed"][int(token)].copy()
        for i, b in enumerate(self.cfg.blocks):
            x = self._block_step(i, b, s, x)
        s.t += 1
        logits = self.st(rms_scale(x, self.eps)[0] * (self.W["lm_head"] @ self.st(x)))
        return logits, s

    def _block_step(self, i, b, s: SeqState, x):
        d = self.d
        # norm(x) W^T: the row in the storage type as the operand, its RMSNorm
        # scale r on the sum
        r, u = rms_scale(x, self.eps)[0], self.st(x)
        if b.kind == "mlp":
            wgu = self.W[f"b{i}.w_gu"]
            g = self.st(r * (wgu[: b.d_ff] @ u))
            up = self.st(r * (wgu[b.d_ff:] @ u))
            m = self.st(gelu(g) * up)
            return x + self.st(self.W[f"b{i}.w_down"] @ m)
        z = self.st(r * (self.W[f"b{i}.w_in"] @ u))
        q, k, v = z[:d], z[d:2 * d], z[2 * d:]
        if b.kind == "fir":
            h = k * v
            taps = self.W[f"b{i}.taps"]                    # [d, L]
            L = b.fir_len
            # newest first: window[j] = h_{t-j}
            window = np.vstack([h[None, :], s.fir[i][::-1]])
            y = np.zeros(d)
            for j in range(L):
                y = y + taps[:, j] * window[j]
            s.fir[i] = np.vstack([s.fir[i], h[None, :]])[1:] if L > 1 else s.fir[i]
            o = self.st(q * y)
        elif b.kind == "iir":
            h = k * v
            lam, res = self.W[f"b{i}.lam"], self.W[f"b{i}.res"]
            s.iir[i] = lam * s.iir[i] + h[:, None]
            y = (res * s.iir[i]).sum(axis=1)
            o = self.st(q * y)
        elif b.kind == "attn":
            H, Dh = b.n_heads, b.head_dim
            qh, kh, vh = q.reshape(H, Dh), k.reshape(H, Dh), v.reshape(H, Dh)
            s.k[i] = np.concatenate([s.k[i], kh[None]], axis=0)
            s.v[i] = np.concatenate([s.v[i], vh[None]], axis=0)
            o = np.zeros((H, Dh))
            for hd in range(H):
                sc = s.k[i][:, hd, :] @ qh[hd] / np.sqrt(Dh)     # keys 0..t
                w = np.exp(sc - sc.max())
                w /= w.sum()
                o[hd] = w @ s.v[i][:, hd, :]
            o = self.st(o.reshape(d))
        else:
            raise ValueError(b.kind)
        return x + self.st(self.W[f"b{i}.w_out"] @ o)

    # -------------------------------------------------------------- block form
    def block(self, state: SeqState, tokens, keep_x: bool = False) -> Pending:
        """Block-verification forward over the candidate tokens (P of them):
        logits for every position and the per-position state. ``state`` is
        not modified."""
        tokens = np.asarray(tokens, dtype=np.int64)
        return self.block_rows(state, self.W["embed"][tokens].copy(), tokens, keep_x)

    def block_rows(self, state: SeqState, X, tokens=None, keep_x: bool = False) -> Pending:
        """The block forward from given input rows X [P, d] (the embedded
        candidates, or a drafter's slot rows)."""
        X = np.array(X, dtype=np.float64)
        if tokens is None:
            tokens = np.zeros(X.shape[0], dtype=np.int64)
        pend = Pending(base=state, tokens=np.asarray(tokens, dtype=np.int64), logits=None)
        for i, b in enumerate(self.cfg.blocks):
            X = self.block_layer(i, b, state, X, pend)
            if keep_x:
                pend.x_out[i] = X.copy()
        pend.logits = self.head(X)
        return pend

    def block_layer(self, i, b, state: SeqState, X, pend: Pending):
        """One residual block over P positions (rows of X) from committed
        ``state``; per-position state goes into ``pend``."""
        d, P = self.d, X.shape[0]
        if b.kind == "mlp":
            wgu = self.W[f"b{i}.w_gu"]
            G = self.st(self.normed_mm(X, wgu[: b.d_ff]))
            Up = self.st(self.normed_mm(X, wgu[b.d_ff:]))
            M = self.st(gelu(G) * Up)
            return X + self.st(self.mm(M, self.W[f"b{i}.w_down"]))
        Z = self.st(self.normed_mm(X, self.W[f"b{i}.w_in"]))
        pend.z[i] = Z
        Q, K, V = Z[:, :d], Z[:, d:2 * d], Z[:, 2 * d:]
        if b.kind == "fir":
            Hh = K * V                                            # [P, d]
            pend.fir_h[i] = Hh
            O = self.st(Q * fir_conv(state.fir[i], Hh, self.W[f"b{i}.taps"]))
        elif b.kind == "iir":
            Hh = K * V
            Y, S = iir_scan(state.iir[i], Hh, self.W[f"b{i}.lam"], self.W[f"b{i}.res"])
            pend.iir_s[i] = S
            O = self.st(Q * Y)
        elif b.kind == "attn":
            H, Dh = b.n_heads, b.head_dim
            Kn, Vn = K.reshape(P, H, Dh), V.reshape(P, H, Dh)
            pend.k_new[i], pend.v_new[i] = Kn, Vn
            Oh = causal_attention(state.k[i], state.v[i], Q.reshape(P, H, Dh), Kn, Vn)
            O = self.st(Oh.reshape(P, d))
        else:
            raise ValueError(b.kind)
        return X + self.st(self.mm(O, self.W[f"b{i}.w_out"]))

    def rollback(self, pend: Pending, n_keep: int) -> SeqState:
        """State sliced to the first ``n_keep`` candidate positions (0..P)."""
        if not 0 <= n_keep <= pend.P:
            raise ValueError("n_keep out of range")
        base = pend.base
        s = base.clone()
        s.t = base.t + n_keep
        for i in base.fir:
            if n_keep:
                s.fir[i] = pend.fir_window(i, n_keep - 1).copy()
        for i in base.iir:
            if n_keep:
                s.iir[i] = pend.iir_s[i][n_keep - 1].copy()
        for i in base.k:
            s.k[i] = np.concatenate([base.k[i], pend.k_new[i][:n_keep]], axis=0)
            s.v[i] = np.concatenate([base.v[i], pend.v_new[i][:n_keep]], axis=0)
        return s

    def prefill(self, tokens, chunk: int = 256):
        """Consume a prompt through the block form in chunks; returns (last
        logits row, committed state)."""
        s = self.empty_state()
        last = None
        tokens = np.asarray(tokens)
        for a in range(0, len(tokens), chunk):
            pend = self.block(s, tokens[a:a + chunk])
            s = self.rollback(pend, pend.P)
            last = pend.logits[-1]
        return last, s
