"""Pins of the oracle's scalar numerics against library routines and closed forms."""
import math

import numpy as np
import pytest
import torch
from scipy.stats import norm

from oracle.numerics import round_bf16, gelu, rmsnorm


def test_round_bf16_matches_torch_conversion():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * s for s in (1e-3, 1.0, 1e3)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(round_bf16(x.astype(np.float64)), ref)


def test_round_bf16_ties_to_even():
    # spacing of bf16 just above 1 is 2^-7
    assert round_bf16(1 + 2.0 ** -8) == 1.0                 # tie -> even mantissa (1.0)
    assert round_bf16(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6   # tie -> even mantissa (2)
    assert round_bf16(1 + 2.0 ** -8 + 2.0 ** -20) == 1 + 2.0 ** -7
    assert round_bf16(-(1 + 2.0 ** -8)) == -1.0
    assert round_bf16(255.5) == 256.0
    assert np.isnan(round_bf16(np.nan)) and round_bf16(np.inf) == np.inf


def test_gelu_is_x_times_normal_cdf():
    x = np.linspace(-6, 6, 1001)
    assert np.allclose(gelu(x), x * norm.cdf(x), rtol=0, atol=1e-15)
    # Phi(1) to 16 digits (standard normal table)
    assert abs(gelu(1.0) - 0.8413447460685429) < 1e-15
    assert gelu(0.0) == 0.0


def test_rmsnorm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 64))
    y = rmsnorm(x, 0.0)
    assert np.allclose(np.sqrt((y ** 2).mean(-1)), 1.0, atol=1e-14)
    assert np.allclose(rmsnorm(7.5 * x, 0.0), y, atol=1e-14)
    # eps enters under the square root: a zero vector stays zero
    assert np.all(rmsnorm(np.zeros(8), 1e-6) == 0)
    v = np.array([3.0, 4.0])
    assert np.allclose(rmsnorm(v, 1.0), v / math.sqrt(12.5 + 1.0))
