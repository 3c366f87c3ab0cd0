"""FP8 weight variant of the oracle (test infrastructure, fp64).

The projection matrices are held as OCP FP8 E4M3 values with one power-of-two
scale per output row; activations, states and accumulation are unchanged.
Reading (the pages name the format, not the scaling): row n keeps
q[n, k] = e4m3(W[n, k] / s[n]) with s[n] the smallest power of two such that
max_k |W[n, k]| <= 448 * s[n], so the division and the scale-back are exact and
the only rounding is e4m3's own (to nearest, ties to even). The effective
weight is q[n, k] * s[n]; the oracle runs the bf16 model with those weights.

Parity pins (tests/test_oracle_fp8.py): round_e4m3 against torch's
float -> float8_e4m3fn conversion, idempotence on every finite E4M3 code,
the scale bounds.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0

# matrices of a block that the FP8 variant stores in E4M3 (the LM head and the
# embedding stay in the model's storage type)
FP8_MATRICES = ("w_in", "w_out", "w_gu", "w_down")


def round_e4m3(x):
    """Nearest E4M3 value (ties to even) as float64.

    E4M3 has a sign, 4 exponent bits (bias 7) and 3 mantissa bits: normal
    values (1 + m/8) * 2**e for e in -6 .. 8 (largest 448), subnormals
    k * 2**-9. A magnitude whose leading bit has weight 2**p is therefore
    quantised to a multiple of 2**max(p - 3, -9). Magnitudes beyond 448 do not
    arise after row scaling and are clamped to 448.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)                       # a = f * 2**e, 0.5 <= f < 1: leading bit 2**(e - 1)
    qe = np.maximum(e - 4, -9)
    q = np.ldexp(np.rint(np.ldexp(a, -qe)), qe)
    return np.copysign(np.minimum(q, E4M3_MAX), x)


def row_scales(W):
    """Per row: the smallest power of two s with max|w| <= 448 * s (1 for a
    zero row). With max|w| = f * 2**e (0.5 <= f < 1) and 448 = 0.875 * 2**9:
    s = 2**(e - 9) if f <= 0.875, else 2**(e - 8)."""
    amax = np.max(np.abs(np.asarray(W, dtype=np.float64)), axis=-1)
    f, e = np.frexp(amax)
    k = np.where(f <= 0.875, e - 9, e - 8)
    return np.where(amax > 0, np.ldexp(1.0, k), 1.0)


def quantize_rows(W):
    """(q, s): E4M3 values of W / s and the row scales s."""
    W = np.asarray(W, dtype=np.float64)
    s = row_scales(W)
    return round_e4m3(W / s[..., None]), s


def fp8_weights(cfg, weights):
    """The model's weights with every block's projection matrices replaced by
    their FP8 effective values q * s (float64); other tensors unchanged."""
    out = {}
    for name, w in weights.items():
        parts = name.split(".")
        if len(parts) == 2 and parts[0].startswith("b") and parts[1] in FP8_MATRICES:
            arr = w.detach().to("cpu").double().numpy() if hasattr(w, "detach") else np.asarray(w, np.float64)
            q, s = quantize_rows(arr)
            out[name] = q * s[:, None]
        else:
            out[name] = w
    return out
