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
