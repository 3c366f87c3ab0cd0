"""Seeded generators for every input of the block-verify path.

Each tensor gets its own generator keyed by (seed, tensor name), so any tensor
can be regenerated alone and in any order. Dense weights, FIR taps and the
embedding are N(0, 0.02) drawn in fp32 and rounded to bf16 (RNE) for bf16
models; IIR poles are U(0.5, 0.99) and residues N(0, 0.1), kept in fp32.
Prompts are i.i.d. uniform over the four DNA letters.

Matrices are drawn with torch generators on the requested device, so large
stacks can be generated directly in device memory; a stack generated on one
device and copied to another carries identical values. Small vectors (draft
distributions, uniforms) are drawn with NumPy PCG64.
"""
from __future__ import annotations

import zlib
from typing import Dict

import numpy as np
import torch

from .configs import ModelConfig, ACGT_IDS, FIR, IIR, ATTN, MLP

WEIGHT_STD = 0.02
RESIDUE_STD = 0.1
MARKOV_STD = 1.0      # drafter transition logits (fp32)
POLE_LO, POLE_HI = 0.5, 0.99


def _key(seed: int, *parts) -> int:
    h = zlib.crc32(("/".join(str(p) for p in parts)).encode())
    return (int(seed) * 0x9E3779B1 + h) & 0x7FFFFFFFFFFFFFFF


def rng_for(seed: int, *parts) -> np.random.Generator:
    """NumPy generator keyed by (seed, *parts)."""
    return np.random.Generator(np.random.PCG64(_key(seed, *parts)))


def _torch_gen(device, seed, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_key(seed, *parts))
    return g


def _normal(shape, std, device, seed, name, store_dtype):
    g = _torch_gen(device, seed, name)
    w = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std
    return w.to(store_dtype)


def weight_names(cfg: ModelConfig):
    """Canonical tensor names and shapes, in library order."""
    d, V = cfg.d_model, cfg.vocab
    out = [("embed", (V, d))]
    for i, b in enumerate(cfg.blocks):
        if b.kind == FIR:
            out += [(f"b{i}.w_in", (3 * d, d)), (f"b{i}.taps", (d, b.fir_len)),
                    (f"b{i}.w_out", (d, d))]
        elif b.kind == IIR:
            out += [(f"b{i}.w_in", (3 * d, d)), (f"b{i}.lam", (d, b.iir_states)),
                    (f"b{i}.res", (d, b.iir_states)), (f"b{i}.w_out", (d, d))]
        elif b.kind == ATTN:
            out += [(f"b{i}.w_in", (3 * d, d)), (f"b{i}.w_out", (d, d))]
        elif b.kind == MLP:
            out += [(f"b{i}.w_gu", (2 * b.d_ff, d)), (f"b{i}.w_down", (d, b.d_ff))]
        else:
            raise ValueError(b.kind)
    out.append(("lm_head", (V, d)))
    if cfg.inject_dim:
        out += [("inject", (d, cfg.inject_dim)), ("pos", (cfg.max_slots, d)), ("markov", (V, V))]
    return out


def make_weights(cfg: ModelConfig, seed: int = 0, device="cpu") -> Dict[str, torch.Tensor]:
    """All canonical weights of ``cfg``.

    Matrices ([rows, cols] row-major, y = x @ W.T) are bf16 tensors for bf16
    models and fp32 for fp32 models. FIR taps ([d, L], tap j multiplies the
    input j steps back) hold bf16-representable values for bf16 models but are
    returned as fp32, as are the IIR poles and residues ([d, N]).
    """
    mat_dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    out = {}
    for name, shape in weight_names(cfg):
        if name.endswith(".lam"):
            g = _torch_gen(device, seed, name)
            out[name] = (torch.rand(shape, generator=g, device=device, dtype=torch.float32)
                         * (POLE_HI - POLE_LO) + POLE_LO)
        elif name.endswith(".res"):
            out[name] = _normal(shape, RESIDUE_STD, device, seed, name, torch.float32)
        elif name.endswith(".taps"):
            out[name] = _normal(shape, WEIGHT_STD, device, seed, name, mat_dtype).float()
        elif name == "markov":
            out[name] = _normal(shape, MARKOV_STD, device, seed, name, torch.float32)
        else:
            out[name] = _normal(shape, WEIGHT_STD, device, seed, name, mat_dtype)
    return out


def prompt_tokens(cfg: ModelConfig, n: int, seed: int = 0, batch: int = 1, tag="prompt") -> np.ndarray:
    """[batch, n] int32 tokens, i.i.d. uniform over the DNA letters."""
    ids = np.asarray(ACGT_IDS(cfg.vocab), dtype=np.int32)
    r = rng_for(seed, tag, n, batch)
    return ids[r.integers(0, 4, size=(batch, n))]


def draft_probs_softmax(shape, vocab: int, seed: int = 0, tag="q") -> np.ndarray:
    """Draft distributions softmax(N(0,1) logits) over the full vocabulary, fp32."""
    r = rng_for(seed, tag, *shape)
    z = r.standard_normal(tuple(shape) + (vocab,))
    e = np.exp(z - z.max(-1, keepdims=True))
    return (e / e.sum(-1, keepdims=True)).astype(np.float32)


def dirichlet_acgt(shape, vocab: int, alpha: float, seed: int = 0, tag="dir") -> np.ndarray:
    """Dirichlet(alpha) distributions over the four DNA letters, embedded in a
    ``vocab``-entry distribution (zero mass elsewhere), fp32."""
    r = rng_for(seed, tag, alpha, *shape)
    p4 = r.dirichlet([alpha] * 4, size=tuple(shape))
    out = np.zeros(tuple(shape) + (vocab,), dtype=np.float32)
    for j, t in enumerate(ACGT_IDS(vocab)):
        out[..., t] = p4[..., j]
    return out


def sample_from(probs: np.ndarray, seed: int, tag="draw") -> np.ndarray:
    """One categorical draw per row of ``probs`` ([..., V]) with a seeded
    inverse-CDF in float64 (used to draw synthetic draft tokens from q)."""
    r = rng_for(seed, tag, *probs.shape)
    u = r.random(probs.shape[:-1])
    c = np.cumsum(probs.astype(np.float64), axis=-1)
    c /= c[..., -1:]
    return (c < u[..., None]).sum(-1).clip(0, probs.shape[-1] - 1).astype(np.int32)


def uniforms(shape, seed: int = 0, tag="u") -> np.ndarray:
    """fp32 uniforms in [0, 1)."""
    return rng_for(seed, tag, *shape).random(tuple(shape), dtype=np.float32)


def synthetic_state(cfg: ModelConfig, t: int, seed: int = 0, device="cpu", std: float = 1.0):
    """A synthetic committed state at context length ``t`` (for long contexts
    that are imported rather than prefilled).

    Returns, per mixer block index: FIR -> {"hist": [L-1, d] fp32, the inputs at
    positions t-L+1 .. t-1, zero where the position is negative};
    IIR -> {"s": [d, N] fp32}; ATTN -> {"k": [t, H, Dh], "v": [t, H, Dh]} in the
    model's storage dtype.
    """
    d = cfg.d_model
    kv_dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    st = {}
    for i, b in enumerate(cfg.blocks):
        if b.kind == FIR:
            h = _normal((b.fir_len - 1, d), std, device, seed, f"st{i}.hist", torch.float32)
            npos = min(b.fir_len - 1, t)
            if npos < b.fir_len - 1:
                h[: b.fir_len - 1 - npos] = 0
            st[i] = {"hist": h}
        elif b.kind == IIR:
            s = _normal((d, b.iir_states), std, device, seed, f"st{i}.s", torch.float32)
            if t == 0:
                s.zero_()
            st[i] = {"s": s}
        elif b.kind == ATTN:
            st[i] = {"k": _normal((t, b.n_heads, b.head_dim), std, device, seed, f"st{i}.k", kv_dtype),
                     "v": _normal((t, b.n_heads, b.head_dim), std, device, seed, f"st{i}.v", kv_dtype)}
    return st


def dyadic_weights(cfg: ModelConfig, seed: int = 0, device="cpu", step_log2: int = 8, span: int = 4):
    """Weights on a coarse dyadic grid for exact-arithmetic checks.

    Matrices hold n * 2**-step_log2 with n uniform in [-span, span] and the
    embedding holds +-1, so the first block's normalised input is +-1 and its
    in-projection outputs are sums that fp32 and fp64 both carry exactly
    (given d * span * 2**-step_log2 < 2**(24 - step_log2)). FIR taps, IIR poles
    and residues are drawn as in ``make_weights``.
    """
    base = make_weights(cfg, seed, device)
    mat_dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    out = {}
    for name, shape in weight_names(cfg):
        if name.endswith((".lam", ".res", ".taps")) or name == "markov":
            out[name] = base[name]
            continue
        g = _torch_gen(device, seed, "dyadic", name)
        if name == "embed":
            w = torch.randint(0, 2, shape, generator=g, device=device).float() * 2 - 1
        else:
            w = torch.randint(-span, span + 1, shape, generator=g, device=device).float() * 2.0 ** -step_log2
        out[name] = w.to(mat_dtype)
    return out
