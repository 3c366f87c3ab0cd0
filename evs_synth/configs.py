"""Model shapes of the synthetic hybrid stacks.

A model is an embedding, a list of pre-norm residual blocks and an untied LM
head. A block is one of: a FIR mixer (depthwise causal filter of ``fir_len``
taps), an IIR mixer (diagonal real modal recurrence with ``iir_states`` modes per
channel), a causal attention mixer (``n_heads`` x ``head_dim`` = d_model) or a
gated-GELU MLP (``d_ff`` hidden units). The hybrid layout follows the
StripedHyena2 description on the EvSpark pages (preprint abstract; GitHub
discussion, "The systems problem"); sizes are the synthetic stand-ins for Evo2 7B.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List

FIR, IIR, ATTN, MLP = "fir", "iir", "attn", "mlp"

# Token ids of the four DNA letters. With a byte vocabulary (>= 256 entries)
# the letters sit at their ASCII codes; with smaller vocabularies they are 0..3.
ACGT_BYTES = (65, 67, 71, 84)


def ACGT_IDS(vocab: int):
    return ACGT_BYTES if vocab >= 256 else (0, 1, 2, 3)


@dataclass(frozen=True)
class Block:
    kind: str
    fir_len: int = 0
    iir_states: int = 0
    n_heads: int = 0
    head_dim: int = 0
    d_ff: int = 0


@dataclass
class ModelConfig:
    name: str
    d_model: int
    vocab: int
    blocks: List[Block] = field(default_factory=list)
    dtype: str = "bf16"          # storage type of weights/activations/KV/logits
    norm_eps: float = 1e-6
    # drafter form (0 = a plain model): width of the injected target hidden
    # state and the number of parallel draft slots (position embeddings)
    inject_dim: int = 0
    max_slots: int = 0

    def weight_bytes(self) -> int:
        """Bytes of the dense matrices (embedding, projections, MLP, LM head)."""
        es = 2 if self.dtype == "bf16" else 4
        d, n = self.d_model, 0
        n += 2 * self.vocab * d
        for b in self.blocks:
            if b.kind in (FIR, IIR, ATTN):
                n += 4 * d * d
            elif b.kind == MLP:
                n += 3 * d * b.d_ff
        return n * es

    def layer_matrix_bytes(self) -> int:
        """Bytes of the per-layer matrices only (no embedding / LM head)."""
        es = 2 if self.dtype == "bf16" else 4
        d, n = self.d_model, 0
        for b in self.blocks:
            if b.kind in (FIR, IIR, ATTN):
                n += 4 * d * d
            elif b.kind == MLP:
                n += 3 * d * b.d_ff
        return n * es


def tiny_c1() -> ModelConfig:
    """Tiny fp32 hybrid stack: FIR(7), IIR(16), attention 4x32, MLP 512; d=128, vocab 4."""
    return ModelConfig("tiny_c1", 128, 4,
                       [Block(FIR, fir_len=7), Block(IIR, iir_states=16),
                        Block(ATTN, n_heads=4, head_dim=32), Block(MLP, d_ff=512)],
                       dtype="f32")


def pair_c2(fir_len: int, d: int = 4096, vocab: int = 512) -> ModelConfig:
    """One IIR + FIR mixer pair at d=4096, bf16 activations and fp32 state."""
    return ModelConfig(f"pair_c2_fir{fir_len}", d, vocab,
                       [Block(IIR, iir_states=16), Block(FIR, fir_len=fir_len)], dtype="bf16")


def hybrid_layer_kinds(n_layers: int):
    """Mixer of each layer: attention on every 8th layer (index % 8 == 7); the
    others cycle FIR-short -> FIR-medium -> IIR."""
    kinds, cyc = [], 0
    for i in range(n_layers):
        if i % 8 == 7:
            kinds.append(ATTN)
        else:
            kinds.append(("fir_s", "fir_m", IIR)[cyc % 3])
            cyc += 1
    return kinds


def stack_7b(n_layers: int = 32, d: int = 4096, d_ff: int = 11008, vocab: int = 512,
             n_heads: int = 32, fir_short: int = 7, fir_medium: int = 128,
             iir_states: int = 16, name: str = "stack_7b") -> ModelConfig:
    """Random-init 32-layer hybrid stack shaped like a 7B model (~13 GB of bf16)."""
    blocks = []
    for k in hybrid_layer_kinds(n_layers):
        if k == "fir_s":
            blocks.append(Block(FIR, fir_len=fir_short))
        elif k == "fir_m":
            blocks.append(Block(FIR, fir_len=fir_medium))
        elif k == IIR:
            blocks.append(Block(IIR, iir_states=iir_states))
        else:
            blocks.append(Block(ATTN, n_heads=n_heads, head_dim=d // n_heads))
        blocks.append(Block(MLP, d_ff=d_ff))
    return ModelConfig(name, d, vocab, blocks, dtype="bf16")


def small_stack(d: int = 256, d_ff: int = 672, vocab: int = 512, head_dim: int = 128,
                fir_medium: int = 128, dtype: str = "bf16") -> ModelConfig:
    """An 8-layer hybrid stack (all mixer kinds, attention at layer 7) small
    enough for the oracle to run in seconds, with every size a few tiles wide."""
    cfg = stack_7b(n_layers=8, d=d, d_ff=d_ff, vocab=vocab, n_heads=d // head_dim,
                   fir_medium=fir_medium, name=f"small_stack_d{d}")
    cfg.dtype = dtype
    return cfg


def drafter_1024(vocab: int = 512, inject_dim: int = 4096, max_slots: int = 16) -> ModelConfig:
    """The gamma-parallel drafter: width 1024, one pre-norm attention (8 x 128)
    + gated-MLP layer (d_ff = 2752, the target's d_ff / d_model ratio of
    2.6875), injected with a ``inject_dim``-wide target hidden state."""
    return ModelConfig("drafter_1024", 1024, vocab, [Block(ATTN, n_heads=8, head_dim=128), Block(MLP, d_ff=2752)],
                       dtype="bf16", inject_dim=inject_dim, max_slots=max_slots)

