"""The weight-read floor kernel (evs_measure_weight_stream; Evo2 discussion
#232, "Regime overlap": the single-stream step is bounded by reading the
weights) reads exactly the packed bytes of the projection it names, each
once. Every thread leaves the XOR of the 32-bit words it loaded, so the XOR
over a workgroup's 512 words equals the XOR of the canonical rows of that
group's output tiles: a fragment lane holds 8 consecutive columns of one row,
so a 32-bit word pairs the same two elements in the packed and the canonical
layout. The small stack's down-projection (K = 672: 21 k-steps, the last of
the 8 wave ranges empty) covers a wave with nothing to read.
"""
import numpy as np
import pytest
import torch

import evs_synth as es
from evs_synth.configs import MLP

from gpu_util import DEV
from attention_dna_lms_amd import evs

pytestmark = pytest.mark.gpu


def xor_rows(w_int32, rows):
    return np.bitwise_xor.reduce(w_int32[rows].reshape(-1))


def cases(cfg):
    """(block, selector, canonical name, tiles per group, rows per tile set)."""
    out = []
    for i, b in enumerate(cfg.blocks):
        if b.kind == MLP:
            out += [(i, evs.EVS_W_GU, f"b{i}.w_gu", 2, b.d_ff), (i, evs.EVS_W_DOWN, f"b{i}.w_down", 1, None)]
        else:
            out += [(i, evs.EVS_W_IN, f"b{i}.w_in", 3, cfg.d_model), (i, evs.EVS_W_OUT, f"b{i}.w_out", 1, None)]
    out.append((-1, evs.EVS_W_LM, "lm_head", 1, None))
    return out


def test_weight_stream_reads_each_group_exactly_once():
    cfg = es.small_stack()
    w = es.make_weights(cfg, seed=301)
    model = evs.Model(cfg, w, device=DEV)
    seen = set()
    for block, which, name, NT, part in cases(cfg):
        key = (which, tuple(w[name].shape))
        if key in seen and which != evs.EVS_W_LM:
            continue                                   # one block of each projection shape
        seen.add(key)
        W = w[name].cpu().contiguous()
        N, K = W.shape
        wi = W.view(torch.int32).numpy()               # [N, K / 2] words
        groups = N // (16 * NT)
        sink = torch.full((groups * 512,), -1, dtype=torch.int32, device=DEV)
        by = evs.evs_measure_weight_stream(model, block, which, sink)
        torch.cuda.synchronize()
        assert by == N * K * 2, name
        got = np.bitwise_xor.reduce(sink.cpu().numpy().reshape(groups, 512), axis=1)
        step = part if part else 0
        want = np.array([xor_rows(wi, [nt * step + g * 16 + r for nt in range(NT) for r in range(16)])
                         for g in range(groups)], dtype=np.int32)
        assert np.array_equal(got, want), name


def test_weight_stream_rejects_bad_arguments():
    cfg = es.small_stack()
    model = evs.Model(cfg, es.make_weights(cfg, seed=302), device=DEV)
    mixer = next(i for i, b in enumerate(cfg.blocks) if b.kind != MLP)
    small = torch.zeros(16, dtype=torch.int32, device=DEV)
    with pytest.raises(evs.EvsError) as e:
        evs.evs_measure_weight_stream(model, mixer, evs.EVS_W_IN, small)
    assert e.value.status == -2                       # EVS_E_RANGE: sink smaller than one word per thread
    sink = torch.zeros(1 << 20, dtype=torch.int32, device=DEV)
    with pytest.raises(evs.EvsError) as e:
        evs.evs_measure_weight_stream(model, mixer, evs.EVS_W_GU, sink)
    assert e.value.status == -1                       # EVS_E_INVALID: a mixer block has no gate/up
    with pytest.raises(evs.EvsError) as e:
        evs.evs_measure_weight_stream(model, len(cfg.blocks), evs.EVS_W_OUT, sink)
    assert e.value.status == -1
