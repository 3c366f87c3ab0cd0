"""Scalar numerics of the oracle (fp64).

Part of the oracle: test infrastructure only (the tests, the smoke check and
the benchmark's CPU-baseline leg may import it; the HIP path never does).

Parity pins (tests/test_oracle_numerics.py):
  round_bf16 — against torch's float->bfloat16 conversion and hand-checked
               tie cases.
  gelu       — against x * Phi(x) from scipy's normal CDF and the tabulated
               value Phi(1).
  rmsnorm    — unit root-mean-square output and scale invariance.
  rms_scale  — the factor rmsnorm multiplies by (same pins).
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf


def round_bf16(x):
    """Round to the nearest bfloat16 value, ties to even; returned as float64.

    bfloat16 keeps 8 significant bits. With x = m * 2**e and 0.5 <= |m| < 1,
    m * 2**8 is rounded to an integer (half to even) and scaled back. Values
    below bfloat16's normal range are rounded as if normal (they do not occur
    in these workloads); infinities and NaN pass through.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def store(x, dtype: str):
    """Value as held in the model's storage type: bf16 rounds, fp32 models keep
    the fp64 value (their casts are the identity in this oracle)."""
    return round_bf16(x) if dtype == "bf16" else np.asarray(x, dtype=np.float64)


def gelu(x):
    """Exact GELU: x * Phi(x) = 0.5 * x * (1 + erf(x / sqrt(2)))."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def rmsnorm(x, eps: float):
    """RMSNorm with unit gain over the last axis: x / sqrt(mean(x^2) + eps)."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rms_scale(x, eps: float):
    """The RMSNorm scale of each row (last axis): 1 / sqrt(mean(x^2) + eps),
    keeping the last axis (length 1) so it broadcasts over the row."""
    x = np.asarray(x, dtype=np.float64)
    return 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
