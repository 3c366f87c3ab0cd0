"""The headline configuration end to end against the oracle: the 32-layer
7B-shaped stack (d = 4096, FIR-7 / FIR-128 / IIR-16 mixers, 32 x 128 attention
every 8th layer, gated MLP d_ff = 11008, vocab 512) at an imported
8192-token state, one gamma = 12 block.

Comparisons (tolerances from the logit bar and readings R18 and R23):
  * teacher forced, layer by layer: the oracle runs block i on the residual
    rows the GPU exported as block i's input, so each comparison sees one
    block's rounding only. The block's output (x_after - x_in) is within
    2^-7 of the oracle's norm-wise. Every filter input h = k v, and every
    K/V row, is within the rounding bound of one bf16 step of the entry plus
    one of its row's rms. Every IIR mode of every position is within 1e-5
    relative of the fp64 recurrence driven by the GPU's own inputs.
  * the LM head on the GPU's final residual rows: within 2e-2 of the oracle.
  * free running through all 64 blocks: the logits within 1.5x the drift the
    oracle's own fp32-accumulation arithmetic shows against its fp64 form;
    greedy tokens equal wherever the oracle's top two logits are apart by
    more than twice the largest change that allows.
  * the verifier (sampling, T = 1, top-4) on the GPU's logits equal to the
    oracle verifier's decisions.
Then a ragged rollback to n_keep in {0, 1, 7, 13} (four copies of the same
sequence): each committed state is the slice of the pending per-position
state, bit for bit.
"""
import numpy as np
import pytest
import torch

import evs_synth as es
from oracle import HybridLM
from oracle.hybrid import Pending, iir_scan
from oracle.verifier import argmax_lowest, verify_sample

from gpu_util import DEV, LOGIT_ATOL, block_verify, import_state, lengths, logit_err, near_tie, rel_close, rollback
from attention_dna_lms_amd import evs

pytestmark = pytest.mark.gpu


def bf16_step(x):
    """Spacing of bf16 values in the binade of |x| (an upper bound on the
    distance from x to either bf16 neighbour)."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.ldexp(1.0, (e - 7).astype(np.int64)), np.ldexp(1.0, -133))


def ulp32(x):
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.ldexp(1.0, (e - 23).astype(np.int64)), np.ldexp(1.0, -149))


def rounding_bound(v):
    """How far a bf16 result may sit from the oracle's value v [rows, n] when
    both round the same sum but their inputs differ by single bf16 roundings:
    one step of the entry itself, plus one step of its row's rms for the
    perturbation of the sum before rounding (an absolute amount, so it
    dominates near zero)."""
    v = np.asarray(v, np.float64)
    rms = np.sqrt(np.mean(v * v, axis=-1, keepdims=True))
    return bf16_step(v) + bf16_step(rms)


def kv_rows(state, block, b, lo, hi):
    k = state.tensor(evs.EVS_ST_K, block)[b, :, lo:hi].permute(1, 0, 2)
    vb = state.tensor(evs.EVS_ST_VT, block)[b]
    v = vb.permute(1, 3, 0, 2).reshape(-1, vb.shape[0], vb.shape[2])[lo:hi]
    return k, v


@pytest.mark.timeout(900)
def test_c3_full_stack_block_verify_against_oracle():
    cfg = es.stack_7b()
    d, V = cfg.d_model, cfg.vocab
    gamma, t0 = 12, 8192
    P = gamma + 1
    keeps = [0, 1, 7, 13]
    B = len(keeps)
    print("C3: weights", flush=True)
    w = es.make_weights(cfg, seed=61, device=DEV)
    model = evs.Model(cfg, w, device=DEV)
    wcpu = {k: v.cpu() for k, v in w.items()}
    del w
    state = evs.State(model, B, t0 + 64, P, device=DEV)
    synth = es.synthetic_state(cfg, t0, seed=62, device=DEV)
    for b in range(B):
        import_state(state, cfg, synth, t0, b)
    synth = {i: {k: v.cpu() for k, v in s.items()} for i, s in synth.items()}
    first = es.prompt_tokens(cfg, 1, seed=63)[0]
    drafts = es.prompt_tokens(cfg, gamma, seed=64)[0]
    cand = np.concatenate([first, drafts]).astype(np.int32)

    # ---------------------------------------------------------- GPU side
    lg, lg_dev = block_verify(model, state, np.tile(cand, (B, 1)))
    for b in range(1, B):
        assert np.array_equal(lg[b], lg[0]), b            # a row never depends on its batch
    # the pending per-position state of sequence 0
    ib = int(state.tensor(evs.EVS_ST_IIR_BUF)[0])
    pend_g = {}
    for i, blk in enumerate(cfg.blocks):
        if blk.kind == "fir":
            ring = state.tensor(evs.EVS_ST_FIR_RING, i)[0]
            pos = torch.as_tensor(np.arange(t0, t0 + P) % ring.shape[0], device=DEV)
            pend_g[i] = ring[pos].double().cpu().numpy()
        elif blk.kind == "iir":
            pend_g[i] = state.tensor(evs.EVS_ST_IIR, i)[0, ib ^ 1, :P].double().cpu().numpy()
        elif blk.kind == "attn":
            k, v = kv_rows(state, i, 0, t0, t0 + P)
            pend_g[i] = (k.double().cpu().numpy(), v.double().cpu().numpy())
    # the residual rows after every block (re-running the same block with the
    # export on: the pending block is discarded and recomputed bit for bit)
    xdst = torch.zeros(B, P, d, dtype=torch.float32, device=DEV)
    x_after = {}
    for i in range(len(cfg.blocks)):
        evs.evs_state_export(state, i, xdst)
        again, _ = block_verify(model, state, np.tile(cand, (B, 1)))
        assert np.array_equal(again, lg), i
        x_after[i] = xdst[0].double().cpu().numpy()
    evs.evs_state_export(state, -1)
    # the verifier on the GPU's logits (sampling, T = 1, top-4) against the oracle verifier
    q = es.dirichlet_acgt((1, gamma), V, 0.5, seed=65, tag="q")
    u = es.uniforms((1, P), seed=66)
    n_acc = torch.zeros(1, dtype=torch.int32, device=DEV)
    nxt = torch.zeros(1, dtype=torch.int32, device=DEV)
    evs.evs_verify_sample(1, gamma, V, lg_dev[:1], evs.EVS_TARGET_LOGITS_BF16, torch.as_tensor(q).to(DEV),
                          torch.as_tensor(drafts[None]).to(DEV), torch.as_tensor(u).to(DEV), 1.0, 4, 0,
                          n_acc, nxt, None)
    torch.cuda.synchronize()
    assert (int(n_acc[0]), int(nxt[0])) == verify_sample(lg[0], q[0], drafts, u[0], 1.0, 4)

    # ------------------------------------------------------- oracle side
    print("C3: oracle weights (fp64)", flush=True)
    orc = HybridLM(cfg, wcpu)
    del wcpu
    ost = orc.import_state(t0, synth)
    print("C3: oracle blocks (teacher forced)", flush=True)
    x_in = orc.W["embed"][cand.astype(np.int64)]
    # the GPU's input rows to block 0 are the same bf16 embedding rows
    for i, blk in enumerate(cfg.blocks):
        tf = Pending(base=ost, tokens=cand, logits=None)
        x_o = orc.block_layer(i, blk, ost, x_in, tf)
        x_g = x_after[i]
        # the block's output (x_after - x_in) norm-wise within 2^-7 of the
        # oracle's: the inputs of its last product are within one bf16 step
        # each (<= 2^-8 relative) and it rounds its own result (<= 2^-8)
        out_o = x_o - x_in
        e_out = np.linalg.norm(x_g - x_o) / np.linalg.norm(out_o)
        print(f"C3: block {i} ({blk.kind}): teacher-forced |d out| / |out| = {e_out:.3g}", flush=True)
        assert e_out <= 2.0 ** -7, (i, e_out)
        if blk.kind in ("fir", "iir"):
            kz, vz = tf.z[i][:, d:2 * d], tf.z[i][:, 2 * d:]
            dk, dv = rounding_bound(kz), rounding_bound(vz)
            hbound = np.abs(kz) * dv + np.abs(vz) * dk + dk * dv
        if blk.kind == "fir":
            h_g = pend_g[i]
            assert np.all(np.abs(h_g - tf.fir_h[i]) <= hbound), i
        elif blk.kind == "iir":
            G = pend_g[i]                                     # [P, d, N] fp32 modes
            lam = orc.W[f"b{i}.lam"]
            s_prev = np.vstack([ost.iir[i][None], G[:-1]])
            h_g = G[:, :, 0] - lam[None, :, 0] * s_prev[:, :, 0]   # the GPU's input, from mode 0
            # every mode of every position follows the recurrence from the
            # committed state driven by the GPU's own input (teacher forced)
            _, S_tf = iir_scan(ost.iir[i], h_g, lam, orc.W[f"b{i}.res"])
            assert rel_close(G, S_tf, 1e-5), i
            # and that input is the oracle's k v within the rounding bound of each
            assert np.all(np.abs(h_g - (kz * vz)) <= hbound + 2 * ulp32(G[:, :, 0])), i
        elif blk.kind == "attn":
            kg, vg = pend_g[i]
            ko, vo = tf.k_new[i].reshape(P, d), tf.v_new[i].reshape(P, d)
            assert np.all(np.abs(kg.reshape(P, d) - ko) <= rounding_bound(ko)), i
            assert np.all(np.abs(vg.reshape(P, d) - vo) <= rounding_bound(vo)), i
        x_in = x_g                                            # the next block starts from the GPU's rows
    # the LM head on the GPU's final residual rows: the 2e-2 bar
    err = logit_err(lg[0], orc.head(x_after[len(cfg.blocks) - 1]))
    print(f"C3: teacher-forced LM head bar value {err:.4g}", flush=True)
    assert err < LOGIT_ATOL, err

    # Free running through all 64 blocks. Single bf16 roundings that differ
    # between any two correct implementations accumulate along the residual
    # stream; their size is measured by the oracle's own arithmetic with fp32
    # accumulators (the precision the GPU accumulates in) against its fp64
    # reference. The GPU must stay within 1.5x of that drift, and agree on
    # the greedy token wherever the oracle's top two logits are further apart
    # than the largest change the bound allows, twice over.
    print("C3: oracle blocks (free running, fp64 and fp32 accumulation)", flush=True)
    pend = orc.block(ost, cand)
    p32 = orc.with_accumulation("f32").block(ost, cand)
    dg, d32 = np.abs(lg[0] - pend.logits), np.abs(p32.logits - pend.logits)
    rg, r32 = np.sqrt(np.mean(dg ** 2)), np.sqrt(np.mean(d32 ** 2))
    print(f"C3: free-running logits vs fp64 oracle: GPU max {dg.max():.4g} rms {rg:.4g}; "
          f"fp32-accumulation oracle max {d32.max():.4g} rms {r32:.4g}", flush=True)
    assert rg <= 1.5 * r32 and dg.max() <= max(LOGIT_ATOL, 1.5 * d32.max()), (rg, r32, dg.max(), d32.max())
    for i in range(P):
        if not near_tie(pend.logits[i], tol=2 * 1.5 * d32.max()):
            assert argmax_lowest(lg[0, i]) == argmax_lowest(pend.logits[i]), i

    # ----------------------------------------------------------- rollback
    rollback(state, keeps)
    assert list(lengths(state)) == [t0 + k for k in keeps]
    for b, k in enumerate(keeps):
        ibb, isl = int(state.tensor(evs.EVS_ST_IIR_BUF)[b]), int(state.tensor(evs.EVS_ST_IIR_SLOT)[b])
        for i, blk in enumerate(cfg.blocks):
            if blk.kind == "fir":
                L = blk.fir_len
                ring = state.tensor(evs.EVS_ST_FIR_RING, i)[b]
                pos = np.arange(t0 + k - (L - 1), t0 + k)
                win = ring[torch.as_tensor(pos % ring.shape[0], device=DEV)].double().cpu().numpy()
                want = np.vstack([synth[i]["hist"].double().numpy(), pend_g[i][:k]])[-(L - 1):]
                assert np.array_equal(win, want), (k, i)
            elif blk.kind == "iir":
                st = state.tensor(evs.EVS_ST_IIR, i)[b, ibb, isl].double().cpu().numpy()
                want = synth[i]["s"].double().numpy() if k == 0 else pend_g[i][k - 1]
                assert np.array_equal(st, want), (k, i)
            elif blk.kind == "attn":
                kg, vg = kv_rows(state, i, b, t0, t0 + k)
                assert np.array_equal(kg.double().cpu().numpy(), pend_g[i][0][:k]), (k, i)
                assert np.array_equal(vg.double().cpu().numpy(), pend_g[i][1][:k]), (k, i)
                kc, vc = kv_rows(state, i, b, t0 - 16, t0)
                assert torch.equal(kc.cpu(), synth[i]["k"][t0 - 16:t0]) and torch.equal(vc.cpu(), synth[i]["v"][t0 - 16:t0])
    assert state.error() == 0
