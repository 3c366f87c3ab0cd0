"""Seeded sweeps over small hybrid stacks with awkward shapes: model widths
whose column-group counts are not multiples of the GEMM's group blocks,
FIR lengths on both sides of the epilogue's register prefetch (1, 128, 129),
IIR mode counts 1..16, every head size, blocks of 1..40 positions and
batches of 1..12 ragged sequences. Each case: every sequence's block logits
against the oracle, against the same sequence run alone (bit for bit), and
after a random ragged rollback the committed state against the solo run."""
import numpy as np
import pytest

import evs_synth as es
from evs_synth.configs import Block, ModelConfig
from oracle import HybridLM

from gpu_util import LOGIT_ATOL, logit_err, DEV, block_verify, lengths, make_engine, prefill, rollback
from test_gpu_long_ragged import committed_equal

pytestmark = pytest.mark.gpu


# (d, blocks, B, P, dtype)
CASES = [
    (96, [Block("fir", fir_len=1), Block("iir", iir_states=1), Block("mlp", d_ff=224)], 3, 5, "bf16"),
    (160, [Block("fir", fir_len=129), Block("attn", n_heads=5, head_dim=32), Block("mlp", d_ff=352)], 5, 13, "bf16"),
    (224, [Block("iir", iir_states=7), Block("fir", fir_len=128), Block("mlp", d_ff=480)], 12, 13, "bf16"),
    (192, [Block("attn", n_heads=3, head_dim=64), Block("iir", iir_states=16), Block("mlp", d_ff=416)], 4, 40, "bf16"),
    (256, [Block("attn", n_heads=2, head_dim=128), Block("fir", fir_len=33), Block("mlp", d_ff=672)], 11, 17, "bf16"),
    (128, [Block("fir", fir_len=7), Block("iir", iir_states=3), Block("attn", n_heads=4, head_dim=32)], 2, 1, "bf16"),
    (96, [Block("iir", iir_states=5), Block("fir", fir_len=64), Block("mlp", d_ff=160)], 6, 9, "f32"),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_random_small_stack(case):
    d, blocks, B, P, dtype = CASES[case]
    cfg = ModelConfig(f"rand{case}", d, 512, blocks, dtype=dtype)
    w = es.make_weights(cfg, seed=400 + case)
    rng = es.rng_for(401 + case, "random-configs")
    plen = [int(n) for n in rng.integers(1, 90, B)]
    prompts = [es.prompt_tokens(cfg, n, seed=402 + 7 * case + b)[0] for b, n in enumerate(plen)]
    cand = es.prompt_tokens(cfg, P, seed=403 + case, batch=B).astype(np.int32)
    keep = rng.integers(0, P + 1, B).astype(np.int32)
    print(f"case {case}: d={d} B={B} P={P} {dtype} prompts={plen} keep={list(keep)}", flush=True)
    max_ctx, max_block = 160, max(P, 16)
    model, state = make_engine(cfg, w, batch=B, max_ctx=max_ctx, max_block=max_block)
    prefill(model, state, prompts)
    lg, _ = block_verify(model, state, cand)
    rollback(state, keep)
    orc = HybridLM(cfg, w)
    atol = LOGIT_ATOL if dtype == "bf16" else 1e-4
    for b in range(B):
        _, ost = orc.prefill(prompts[b], chunk=max_block)
        ref = orc.block(ost, cand[b]).logits
        err = logit_err(lg[b], ref) if dtype == "bf16" else float(np.max(np.abs(lg[b] - ref)))
        assert err < atol, (b, err)
        m1, s1 = make_engine(cfg, w, batch=1, max_ctx=max_ctx, max_block=max_block)
        prefill(m1, s1, [prompts[b]])
        one, _ = block_verify(m1, s1, cand[b:b + 1])
        assert np.array_equal(one[0], lg[b]), b
        rollback(s1, keep[b:b + 1])
        assert lengths(s1)[0] == lengths(state)[b] == plen[b] + keep[b]
        assert committed_equal(cfg, state, b, s1, 0), b
    assert state.error() == 0
