"""Pins of the oracle's hybrid stack: mixer ops against library routines and
closed forms, hand-worked stacks, and the invariants the pages fix
(block == sequential, rollback == replay, causal prefix, identity drafter)."""
import math

import numpy as np
import pytest
import torch
from scipy.signal import lfilter
from scipy.stats import norm

import evs_synth as es
from evs_synth.configs import Block, ModelConfig
from oracle import HybridLM, fir_conv, iir_scan, causal_attention, native_greedy, spec_round, replay
from oracle.verifier import argmax_lowest


# ----------------------------------------------------------------- mixer ops
@pytest.mark.parametrize("L,P,t_hist", [(7, 13, 0), (7, 13, 6), (128, 5, 127), (1, 4, 0)])
def test_fir_conv_matches_lfilter(L, P, t_hist):
    rng = np.random.default_rng(L * 100 + P)
    d = 5
    hist = np.zeros((L - 1, d))
    if t_hist:
        hist[-t_hist:] = rng.standard_normal((t_hist, d))
    Hh = rng.standard_normal((P, d))
    taps = rng.standard_normal((d, L))
    Y = fir_conv(hist, Hh, taps)
    for c in range(d):
        full = np.concatenate([hist[:, c], Hh[:, c]])
        ref = lfilter(taps[c], [1.0], full)[L - 1:]
        assert np.allclose(Y[:, c], ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("P,N", [(13, 16), (1, 4), (40, 3)])
def test_iir_scan_matches_impulse_response(P, N):
    """y_p = sum_n res lam^(p+1) s0 + sum_{j<=p} (sum_n res lam^j) h_{p-j}."""
    rng = np.random.default_rng(P * 7 + N)
    d = 6
    lam = rng.uniform(0.5, 0.99, (d, N))
    res = rng.normal(0, 0.1, (d, N))
    s0 = rng.standard_normal((d, N))
    Hh = rng.standard_normal((P, d))
    Y, S = iir_scan(s0, Hh, lam, res)
    for c in range(d):
        kern = np.array([(res[c] * lam[c] ** j).sum() for j in range(P)])
        free = np.array([(res[c] * lam[c] ** (p + 1) * s0[c]).sum() for p in range(P)])
        ref = np.convolve(Hh[:, c], kern)[:P] + free
        assert np.allclose(Y[:, c], ref, rtol=1e-10, atol=1e-12)
        # the state after position p is the mode-wise closed form as well
        for n in range(N):
            sref = lam[c, n] ** np.arange(1, P + 1) * s0[c, n] + np.convolve(Hh[:, c], lam[c, n] ** np.arange(P))[:P]
            assert np.allclose(S[:, c, n], sref, rtol=1e-10, atol=1e-12)


def test_attention_single_key_returns_value():
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((1, 2, 8)) for _ in range(3))
    O = causal_attention(np.zeros((0, 2, 8)), np.zeros((0, 2, 8)), q, k, v)
    assert np.allclose(O, v)


def test_attention_zero_query_averages_visible_values():
    """q = 0 gives uniform weights over exactly the keys at positions <= t+p."""
    rng = np.random.default_rng(4)
    t, P, H, Dh = 5, 4, 3, 8
    Kc, Vc = rng.standard_normal((t, H, Dh)), rng.standard_normal((t, H, Dh))
    Kn, Vn = rng.standard_normal((P, H, Dh)), rng.standard_normal((P, H, Dh))
    O = causal_attention(Kc, Vc, np.zeros((P, H, Dh)), Kn, Vn)
    Va = np.concatenate([Vc, Vn])
    for p in range(P):
        assert np.allclose(O[p], Va[: t + p + 1].mean(0))


def test_attention_two_keys_is_logistic_in_scaled_score():
    Dh = 4
    q = np.array([[[1.0, 2.0, 0.0, -1.0]]])
    k0 = np.array([[[0.5, 0.0, 1.0, 0.0]]])
    k1 = np.array([[[0.0, 1.0, 0.0, 2.0]]])
    v0 = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    v1 = np.array([[[0.0, 1.0, 0.0, 0.0]]])
    O = causal_attention(k0, v0, q, k1, v1)
    a = 1.0 / (1.0 + math.exp(-(0.5 - 0.0) / math.sqrt(Dh)))   # q.k0 = 0.5, q.k1 = 0
    assert np.allclose(O[0, 0], [a, 1 - a, 0, 0])


# ------------------------------------------------------- hand-worked stacks
def _cfg(d, V, blocks, eps=0.0):
    return ModelConfig("hand", d, V, blocks, dtype="f32", norm_eps=eps)


def test_hand_worked_fir_mixer_wiring():
    """d=2, FIR with one tap: q|k|v split order, h = k v, o = q y, residual and
    final norm worked out by hand."""
    cfg = _cfg(2, 2, [Block("fir", fir_len=1)])
    W = {"embed": np.array([[1.0, 1.0], [0.0, 0.0]]),
         "b0.w_in": np.array([[1, 0], [0, 2], [3, 0], [0, 1], [0.5, 0], [0, -1]], float),
         "b0.taps": np.array([[2.0], [1.0]]),
         "b0.w_out": np.eye(2),
         "lm_head": np.eye(2)}
    m = HybridLM(cfg, W)
    logits, _ = m.step(m.empty_state(), 0)
    # u = [1,1]; q=[1,2], k=[3,1], v=[0.5,-1]; h=[1.5,-1]; y=[3,-1]; o=[3,-2]; x=[4,-1]
    assert np.allclose(logits, np.array([4.0, -1.0]) / math.sqrt(8.5))


def test_hand_worked_fir_positions():
    """d=1 with three taps: y_t picks up the inputs of the current and two
    previous positions, with zero before position 0."""
    cfg = _cfg(1, 2, [Block("fir", fir_len=3)])
    W = {"embed": np.array([[2.0], [-1.0]]), "b0.w_in": np.array([[1.0], [1.0], [1.0]]),
         "b0.taps": np.array([[0.5, 0.25, 0.125]]), "b0.w_out": np.array([[1.0]]),
         "lm_head": np.array([[1.0], [-1.0]])}
    m = HybridLM(cfg, W)
    pend = m.block(m.empty_state(), [0, 1, 0, 0])
    # u = sign(x) = +-1, h = u^2 = 1; y = 0.5, 0.75, 0.875, 0.875; x' = x + u y
    xs = np.array([2 + 0.5, -1 - 0.75, 2 + 0.875, 2 + 0.875])
    assert np.allclose(pend.logits[:, 0], np.sign(xs))
    assert np.allclose(pend.fir_h[0][:, 0], 1.0)


def test_hand_worked_iir_recurrence():
    """d=1, one mode with pole 0.5 and residue 1: y_0 = h, y_1 = 1.5 h, y_2 = 1.75 h."""
    cfg = _cfg(1, 1, [Block("iir", iir_states=1)])
    W = {"embed": np.array([[3.0]]), "b0.w_in": np.array([[1.0], [2.0], [0.5]]),
         "b0.lam": np.array([[0.5]]), "b0.res": np.array([[1.0]]),
         "b0.w_out": np.array([[1.0]]), "lm_head": np.array([[1.0]])}
    m = HybridLM(cfg, W)
    pend = m.block(m.empty_state(), [0, 0, 0])
    # u = 1, q = 1, h = k v = 1: s = 1, 1.5, 1.75
    assert np.allclose(pend.iir_s[0][:, 0, 0], [1.0, 1.5, 1.75])


def test_hand_worked_attention_uniform_mean():
    """W_q = 0 makes every query attend uniformly: the second position's output
    is the mean of both positions' values."""
    cfg = _cfg(2, 2, [Block("attn", n_heads=1, head_dim=2)])
    W = {"embed": np.array([[1.0, 1.0], [1.0, -1.0]]),
         "b0.w_in": np.array([[0, 0], [0, 0], [1, 0], [0, 1], [2, 0], [0, 4]], float),
         "b0.w_out": np.eye(2), "lm_head": np.eye(2)}
    m = HybridLM(cfg, W)
    pend = m.block(m.empty_state(), [0, 1], keep_x=True)
    # v_0 = [2, 4], v_1 = [2, -4]; out_0 = v_0, out_1 = mean = [2, 0]
    assert np.allclose(pend.x_out[0][0], [1 + 2, 1 + 4])
    assert np.allclose(pend.x_out[0][1], [1 + 2, -1 + 0])


def test_hand_worked_mlp_wiring():
    """Gate rows come first in W_gu: m = gelu(gate) * up; x += m W_down^T."""
    cfg = _cfg(2, 2, [Block("mlp", d_ff=1)])
    W = {"embed": np.array([[1.0, 1.0], [0.0, 0.0]]),
         "b0.w_gu": np.array([[1.0, 0.0], [0.0, 2.0]]),
         "b0.w_down": np.array([[1.0], [0.0]]), "lm_head": np.eye(2)}
    m = HybridLM(cfg, W)
    logits, _ = m.step(m.empty_state(), 0)
    a = 1 + 2 * norm.cdf(1.0)                      # gate 1, up 2 -> 2 * gelu(1) = 2 Phi(1)
    assert np.allclose(logits, np.array([a, 1.0]) / math.sqrt((a * a + 1) / 2))


# -------------------------------------------------------------- invariants
def _tiny_bf16():
    return ModelConfig("tiny_bf16", 64, 16,
                       [Block("fir", fir_len=7), Block("mlp", d_ff=96), Block("iir", iir_states=4),
                        Block("attn", n_heads=2, head_dim=32), Block("fir", fir_len=12),
                        Block("mlp", d_ff=64)], dtype="bf16")


@pytest.fixture(scope="module", params=["c1", "bf16"])
def model(request):
    cfg = es.tiny_c1() if request.param == "c1" else _tiny_bf16()
    return HybridLM(cfg, es.make_weights(cfg, seed=0))


def _prefix_state(m, n=9, seed=0):
    toks = es.prompt_tokens(m.cfg, n, seed=seed)[0]
    _, s = m.prefill(toks, chunk=4)
    return s


def _close(a, b, rtol):
    scale = np.abs(b).max() + 1e-300
    return np.abs(a - b).max() <= rtol * scale


def test_block_equals_sequential_steps(model):
    """Block verify logits == gamma+1 sequential single-token decode steps."""
    s0 = _prefix_state(model)
    cand = es.prompt_tokens(model.cfg, 6, seed=5)[0]
    pend = model.block(s0, cand)
    s = s0
    for i, tok in enumerate(cand):
        lg, s = model.step(s, tok)
        assert _close(pend.logits[i], lg, 1e-9), i


def test_rollback_equals_replay_for_every_k(model):
    """rollback(k) == the state after k sequential steps from the snapshot."""
    s0 = _prefix_state(model, seed=1)
    cand = es.prompt_tokens(model.cfg, 5, seed=6)[0]
    pend = model.block(s0, cand)
    for k in range(len(cand) + 1):
        a = model.rollback(pend, k)
        b = replay(model, s0, cand[:k])
        assert a.t == b.t == s0.t + k
        for i in a.fir:
            assert _close(a.fir[i], b.fir[i], 1e-12)
        for i in a.iir:
            assert _close(a.iir[i], b.iir[i], 1e-9)
        for i in a.k:
            assert a.k[i].shape == b.k[i].shape and _close(a.k[i], b.k[i], 1e-9)
            assert _close(a.v[i], b.v[i], 1e-9)
        # continuing from either state gives the same next logits
        la, _ = model.step(a, 1)
        lb, _ = model.step(b, 1)
        assert _close(la, lb, 1e-9)


def test_rollback_zero_restores_pre_block_state(model):
    s0 = _prefix_state(model, seed=2)
    pend = model.block(s0, es.prompt_tokens(model.cfg, 4, seed=7)[0])
    r = model.rollback(pend, 0)
    assert r.t == s0.t
    for i in s0.fir:
        assert np.array_equal(r.fir[i], s0.fir[i])
    for i in s0.iir:
        assert np.array_equal(r.iir[i], s0.iir[i])
    for i in s0.k:
        assert np.array_equal(r.k[i], s0.k[i]) and np.array_equal(r.v[i], s0.v[i])
    # verifying the same block again gives identical outputs (deterministic)
    pend2 = model.block(r, pend.tokens)
    assert np.array_equal(pend.logits, pend2.logits)


def test_causal_prefix_shorter_block(model):
    """The first gamma'+1 logits and states of a gamma-block equal a gamma'-block's."""
    s0 = _prefix_state(model, seed=3)
    cand = es.prompt_tokens(model.cfg, 7, seed=8)[0]
    full = model.block(s0, cand)
    for gp in (0, 2, 5):
        short = model.block(s0, cand[: gp + 1])
        assert _close(full.logits[: gp + 1], short.logits, 1e-12)
        for i in full.iir_s:
            assert _close(full.iir_s[i][: gp + 1], short.iir_s[i], 1e-12)


def test_identity_drafter_accepts_everything_greedy(model):
    """Drafts = the native greedy continuation: every draft is accepted and the
    speculative output equals native decoding token for token."""
    s0 = _prefix_state(model, seed=4)
    x0 = 2
    gamma, rounds = 4, 3
    native, _ = native_greedy(model, s0, x0, gamma * rounds + rounds)
    s, x, out, pos = s0, x0, [], 0
    for _ in range(rounds):
        drafts = native[pos: pos + gamma]
        n_acc, nxt, s, _ = spec_round(model, s, x, drafts, greedy=True)
        assert n_acc == gamma
        out += list(drafts) + [nxt]
        pos += gamma + 1
        x = nxt
    assert out == list(native[: len(out)])


def test_greedy_spec_with_bad_drafter_matches_native(model):
    """A drafter that is often wrong still yields the native greedy sequence."""
    s0 = _prefix_state(model, seed=5)
    x0 = 1
    native, _ = native_greedy(model, s0, x0, 12)
    rng = np.random.default_rng(9)
    s, x, out = s0, x0, []
    while len(out) < 12:
        drafts = rng.integers(0, model.cfg.vocab, 3)
        n_acc, nxt, s, _ = spec_round(model, s, x, drafts, greedy=True)
        out += list(drafts[:n_acc]) + [nxt]
        x = nxt
    assert out[:12] == list(native)


def test_oracle_is_deterministic():
    cfg = _tiny_bf16()
    a = HybridLM(cfg, es.make_weights(cfg, seed=3)).block(HybridLM(cfg, es.make_weights(cfg, seed=3)).empty_state(), [1, 2, 3])
    b = HybridLM(cfg, es.make_weights(cfg, seed=3)).block(HybridLM(cfg, es.make_weights(cfg, seed=3)).empty_state(), [1, 2, 3])
    assert np.array_equal(a.logits, b.logits)


def test_bf16_storage_points_are_bf16_values():
    cfg = _tiny_bf16()
    m = HybridLM(cfg, es.make_weights(cfg, seed=0))
    pend = m.block(m.empty_state(), [1, 2, 3, 4])
    as_bf = torch.from_numpy(pend.logits.astype(np.float32)).to(torch.bfloat16).double().numpy()
    assert np.array_equal(as_bf, pend.logits)
    for i in pend.k_new:
        k = pend.k_new[i].astype(np.float32)
        assert np.array_equal(torch.from_numpy(k).to(torch.bfloat16).float().numpy(), k)


def test_normed_product_reads_the_bf16_row_and_scales_the_sum():
    """Reading R3: norm(x) W^T = r (st(x) W^T) with r = 1 / sqrt(mean(x^2) +
    eps): the residual row rounded to bf16 is the operand and r scales the sum,
    in the LM head as in the blocks. Hand-worked: x = [1, 1 + 2^-8, 1, 2]
    rounds to [1, 1, 1, 2] (1 + 2^-8 is the tie between 1 and 1 + 2^-7; ties
    go to the even one) and has r = 1 / sqrt(7.00783 / 4) = 0.75551. Head row
    [1, -1, 0, 0]: r (1 - 1) = 0. Rounding x r first would give 0.75391 -
    0.75781 = -2^-8 (0.75551 and 0.75846 lie 193.4 and 194.2 steps of 2^-8 up),
    and no rounding at all -0.00295. Head row [0, 0, 0, 1]: st(2 r) =
    st(1.51101) = 1.5078125 (step 2^-7)."""
    from evs_synth.configs import ModelConfig
    cfg = ModelConfig("norm_pin", 4, 2, [], dtype="bf16")
    w = {"embed": np.array([[1.0, 1 + 2.0 ** -8, 1, 2], [1, 1, 1, 1]]),
         "lm_head": np.array([[1.0, -1, 0, 0], [0, 0, 0, 1]])}
    orc = HybridLM(cfg, w)
    want = [0.0, 1.5078125]
    assert list(orc.block(orc.empty_state(), [0]).logits[0]) == want
    assert list(orc.step(orc.empty_state(), 0)[0]) == want
    assert list(HybridLM(cfg, w, accumulate="f32").block(orc.empty_state(), [0]).logits[0]) == want
