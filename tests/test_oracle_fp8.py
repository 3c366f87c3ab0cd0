"""Pins of the oracle's FP8 E4M3 quantiser against torch's float8_e4m3fn type
(an independent implementation of the same format) and the scaling rule."""
import numpy as np
import torch

from oracle.fp8 import E4M3_MAX, quantize_rows, round_e4m3, row_scales


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_round_e4m3_matches_torch_conversion():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(40000) * s for s in (1e-3, 0.05, 1.0, 30.0)]
                       + [rng.uniform(-448, 448, 20000)]).astype(np.float32)
    assert np.array_equal(round_e4m3(x.astype(np.float64)), _torch_e4m3(x))


def test_round_e4m3_ties_and_subnormals():
    # ties between neighbours go to the even code, in every binade and below
    for p in range(-9, 9):
        q = 2.0 ** max(p - 3, -9)
        base = np.arange(0, 16) * q + (2.0 ** p if p >= -6 else 0.0)
        mid = (base[:-1] + base[1:]) / 2
        mid = mid[(mid < E4M3_MAX) & (mid > 0)]
        assert np.array_equal(round_e4m3(mid), _torch_e4m3(mid)), p
    assert round_e4m3(2.0 ** -10) == 0.0               # half the smallest subnormal -> 0 (even)
    assert round_e4m3(3 * 2.0 ** -10) == 2 * 2.0 ** -9  # 1.5 subnormal steps -> 2 (even)
    assert round_e4m3(-0.0) == 0.0 and np.signbit(round_e4m3(-0.0))


def test_every_finite_code_is_a_fixed_point():
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = codes[np.isfinite(codes)]
    assert finite.size == 254                          # two NaN codes, no infinities
    assert np.array_equal(round_e4m3(finite), finite)
    assert finite.max() == E4M3_MAX and np.min(finite[finite > 0]) == 2.0 ** -9


def test_row_scales_are_the_smallest_fitting_powers_of_two():
    rng = np.random.default_rng(4)
    # fp32 values, so W / s is exact in fp32 as well (as for bf16 model weights)
    W = (rng.standard_normal((300, 64)) * np.exp(rng.uniform(-12, 12, (300, 1)))).astype(np.float32).astype(np.float64)
    W[7] = 0.0
    W[11, :] = 448.0 * 2.0 ** -5                        # exactly at the bound
    s = row_scales(W)
    m, e = np.frexp(s)
    assert np.all(m == 0.5)                            # powers of two
    amax = np.abs(W).max(axis=1)
    nz = amax > 0
    assert np.all(amax[nz] <= E4M3_MAX * s[nz])
    assert np.all(amax[nz] > E4M3_MAX * s[nz] / 2)     # half the scale would not fit
    assert s[7] == 1.0 and s[11] == 2.0 ** -5
    q, s2 = quantize_rows(W)
    assert np.array_equal(s, s2)
    assert np.array_equal(q, _torch_e4m3((W / s[:, None]).astype(np.float32)))
    assert np.all(np.abs(q) <= E4M3_MAX)


# Hand-worked rows (values checked by hand, not by the quantiser):
#   row 0 = [0.0103, 0.02, -0.0105, 0]: max 0.02 = 0.64 * 2^-5, so s = 2^-14
#     (448 * 2^-14 = 0.0273 fits, 224 * 2^-14 = 0.0137 does not); scaled values
#     168.76, 327.68, -172.03, 0 round in E4M3 steps of 16, 32, 16 to 176, 320,
#     -176, 0 -> [0.0107421875, 0.01953125, -0.0107421875, 0].
#   row 1 = [300, -0.5, 0.25, 1.3]: max 300 = 0.586 * 2^9, so s = 1; 300 rounds
#     in steps of 32 to 288, 1.3 in steps of 1/8 to 1.25 -> [288, -0.5, 0.25, 1.25].
# A column-wise scale would put column 0's 0.0103 on the subnormal grid of
# column max 300 (steps of 2^-9) and give 0.009765625 instead.
HAND_ROWS = np.array([[0.0103, 0.02, -0.0105, 0.0], [300.0, -0.5, 0.25, 1.3]])
HAND_EFFECTIVE = np.array([[0.0107421875, 0.01953125, -0.0107421875, 0.0], [288.0, -0.5, 0.25, 1.25]])


def _two_block_weights():
    """A [FIR(3), MLP(2)] model at d = 4, vocab 6, as float64 arrays: every
    matrix starts with the hand-worked rows, the rest random."""
    from evs_synth.configs import Block, ModelConfig
    cfg = ModelConfig("fp8_pin", 4, 6, [Block("fir", fir_len=3), Block("mlp", d_ff=2)], dtype="bf16")
    rng = np.random.default_rng(11)
    shapes = {"embed": (6, 4), "b0.w_in": (12, 4), "b0.taps": (4, 3), "b0.w_out": (4, 4),
              "b1.w_gu": (4, 4), "b1.w_down": (4, 2), "lm_head": (6, 4)}
    w = {}
    for name, (r, c) in shapes.items():
        a = rng.standard_normal((r, c)) * np.exp(rng.uniform(-6, 3, (r, 1)))
        if c == 4 and name != "b0.taps":
            a[:2] = HAND_ROWS
        # fp32 values (as bf16 model weights are), so W / s is exact in fp32 and
        # torch's fp32 -> e4m3 conversion rounds once
        w[name] = a.astype(np.float32).astype(np.float64)
    return cfg, w


def test_fp8_weights_changes_only_block_projections_row_by_row():
    from oracle.fp8 import fp8_weights
    cfg, w = _two_block_weights()
    out = fp8_weights(cfg, w)
    assert set(out) == set(w)
    # the embedding, LM head and FIR taps pass through untouched (their hand
    # rows are not E4M3 values, so quantising them would show)
    for name in ("embed", "lm_head", "b0.taps"):
        assert np.array_equal(np.asarray(out[name]), w[name]), name
    assert not np.array_equal(round_e4m3(HAND_ROWS), HAND_ROWS)
    for name in ("b0.w_in", "b0.w_out", "b1.w_gu"):
        assert np.array_equal(out[name][:2], HAND_EFFECTIVE), name
    assert not np.array_equal(np.asarray(w['embed'][:2]), HAND_EFFECTIVE)
    # every row of every projection (w_down has 2 columns: no hand rows):
    # e4m3(W[n] / s_n) * s_n with s_n from that row alone, e4m3 by torch
    for name in ("b0.w_in", "b0.w_out", "b1.w_gu", "b1.w_down"):
        W = w[name]
        for n in range(W.shape[0]):
            amax = np.abs(W[n]).max()
            s = 2.0 ** np.ceil(np.log2(amax / E4M3_MAX))     # smallest power of two with amax <= 448 s
            expect = _torch_e4m3(W[n] / s) * s
            assert np.array_equal(out[name][n], expect), (name, n)
