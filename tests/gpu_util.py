"""Helpers for the GPU parity tests: run the HIP library through its C ABI and
bring its outputs and per-position state back in the oracle's terms."""
import numpy as np
import torch

from attention_dna_lms_amd import evs

DEV = "cuda"

# bf16 logits: within 2e-2 absolute of the oracle's (bf16-rounded) value, or
# exactly one bf16 step from it. A step is 2^-5 = 0.03125 at |b| in [4, 8),
# so at those magnitudes a one-step rounding flip of an honest fp32 result is
# the only allowance beyond 2e-2; below |b| = 4 a step is already < 2e-2.
LOGIT_ATOL = 2e-2


def _bf16_order(x):
    """bf16 values as integers in their total order (adjacent values differ by
    one), and whether each value is exactly representable in bf16."""
    f = np.asarray(x, np.float64).astype(np.float32)
    bits = f.view(np.uint32)
    exact = ((bits & 0xFFFF) == 0) & (f.astype(np.float64) == np.asarray(x, np.float64))
    hi = (bits >> 16).astype(np.int64)
    mag = hi & 0x7FFF
    return np.where(hi & 0x8000, -mag, mag), exact


def logit_err(a, b):
    """Largest |a - b| over the entries where a is not exactly one bf16 step
    from b (b: the oracle's bf16 logits; a: the GPU's). An entry one step away
    counts as 0 whatever the step's size; every other entry counts its full
    difference, so `logit_err(a, b) < LOGIT_ATOL` is the bar stated above."""
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    oa, ea = _bf16_order(a)
    ob, eb = _bf16_order(b)
    one_step = ea & eb & (np.abs(oa - ob) == 1)
    diff = np.abs(a - b)
    return float(np.max(np.where(one_step, 0.0, diff)))


def near_tie(row, tol=2 * LOGIT_ATOL):
    """The oracle's two largest logits of a row are within `tol`."""
    s = np.sort(np.asarray(row, np.float64))[::-1]
    return s[0] - s[1] <= tol


def make_engine(cfg, weights, batch=1, max_ctx=1024, max_block=16):
    model = evs.Model(cfg, weights, device=DEV)
    state = evs.State(model, batch, max_ctx, max_block, device=DEV)
    torch.cuda.synchronize()
    return model, state


def storage_dtype(cfg):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def prefill(model, state, prompts):
    """prompts: list of int arrays (one per sequence). Returns last logits [B, V] (fp64 numpy)."""
    cfg = model.cfg
    flat = np.concatenate([np.asarray(p, np.int32) for p in prompts]) if len(prompts) else np.zeros(0, np.int32)
    offs = np.concatenate([[0], np.cumsum([len(p) for p in prompts])]).astype(np.int32)
    tok = torch.from_numpy(flat).to(DEV)
    last = torch.zeros(len(prompts), cfg.vocab, dtype=storage_dtype(cfg), device=DEV)
    evs.evs_prefill(model, state, tok, offs, last)
    torch.cuda.synchronize()
    return last.double().cpu().numpy()


def block_verify(model, state, cand):
    """cand: [B, P] int array. Returns logits [B, P, V] fp64 numpy (and the device tensor)."""
    cfg = model.cfg
    c = torch.as_tensor(np.asarray(cand, np.int32)).to(DEV)
    B, P = c.shape
    lg = torch.empty(B, P, cfg.vocab, dtype=storage_dtype(cfg), device=DEV)
    evs.evs_block_verify(model, state, c, P - 1, lg)
    torch.cuda.synchronize()
    return lg.double().cpu().numpy(), lg


def rollback(state, n_keep):
    nk = None if n_keep is None else torch.as_tensor(np.asarray(n_keep, np.int32)).to(DEV)
    evs.evs_rollback(state, nk)
    torch.cuda.synchronize()


def lengths(state):
    return state.tensor(evs.EVS_ST_T).cpu().numpy().copy()


def snapshot(state, cfg, b=0):
    """Committed state of sequence b in oracle terms: FIR windows [L-1, d],
    IIR modes [d, N], K/V rows [t, H, Dh] (all fp64)."""
    t = int(state.tensor(evs.EVS_ST_T)[b])
    ib = int(state.tensor(evs.EVS_ST_IIR_BUF)[b])
    isl = int(state.tensor(evs.EVS_ST_IIR_SLOT)[b])
    out = {"t": t, "fir": {}, "iir": {}, "k": {}, "v": {}}
    for i, blk in enumerate(cfg.blocks):
        if blk.kind == "fir":
            ring = state.tensor(evs.EVS_ST_FIR_RING, i)[b]
            R = ring.shape[0]
            pos = np.arange(t - (blk.fir_len - 1), t)
            win = ring[torch.as_tensor(pos % R, device=DEV)].double().cpu().numpy()
            win[pos < 0] = 0
            out["fir"][i] = win
        elif blk.kind == "iir":
            st = state.tensor(evs.EVS_ST_IIR, i)[b]
            out["iir"][i] = np.zeros(st.shape[-2:]) if isl < 0 else st[ib, isl].double().cpu().numpy()
        elif blk.kind == "attn":
            out["k"][i] = state.tensor(evs.EVS_ST_K, i)[b, :, :t].permute(1, 0, 2).double().cpu().numpy()
            vb = state.tensor(evs.EVS_ST_VT, i)[b]                  # [H, cap/16, Dh, 16]
            out["v"][i] = vb.permute(1, 3, 0, 2).reshape(-1, vb.shape[0], vb.shape[2])[:t].double().cpu().numpy()
    return out


def pending_iir(state, block, P, b=0):
    """Per-position IIR modes [P, d, N] written by the pending block."""
    ib = int(state.tensor(evs.EVS_ST_IIR_BUF)[b])
    return state.tensor(evs.EVS_ST_IIR, block)[b, ib ^ 1, :P].double().cpu().numpy()


def import_state(state, cfg, synth, t, b=0):
    """Write a synthetic committed state (evs_synth.synthetic_state) for sequence b."""
    state.tensor(evs.EVS_ST_T)[b] = t
    state.tensor(evs.EVS_ST_IIR_BUF)[b] = 0
    state.tensor(evs.EVS_ST_IIR_SLOT)[b] = 0
    for i, blk in enumerate(cfg.blocks):
        if blk.kind == "fir":
            ring = state.tensor(evs.EVS_ST_FIR_RING, i)[b]
            R = ring.shape[0]
            pos = np.arange(t - (blk.fir_len - 1), t)
            ok = pos >= 0
            idx = torch.as_tensor(pos[ok] % R, device=DEV)
            ring[idx] = synth[i]["hist"][torch.as_tensor(np.nonzero(ok)[0])].to(DEV)
        elif blk.kind == "iir":
            state.tensor(evs.EVS_ST_IIR, i)[b, 0, 0] = synth[i]["s"].to(DEV)
        elif blk.kind == "attn":
            state.tensor(evs.EVS_ST_K, i)[b, :, :t] = synth[i]["k"].to(DEV).permute(1, 0, 2)
            vb = state.tensor(evs.EVS_ST_VT, i)[b]                  # [H, cap/16, Dh, 16]
            nb = (t + 15) // 16
            v = torch.zeros(nb * 16, vb.shape[0], vb.shape[2], dtype=vb.dtype, device=DEV)
            v[:t] = synth[i]["v"].to(DEV)
            vb[:, :nb] = v.reshape(nb, 16, vb.shape[0], vb.shape[2]).permute(2, 0, 3, 1)
    torch.cuda.synchronize()


def rel_close(a, b, rtol=1e-5):
    """|a - b| <= rtol * (|b| + rms(b)) elementwise."""
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    rms = np.sqrt(np.mean(b * b)) if b.size else 0.0
    return bool(np.all(np.abs(a - b) <= rtol * (np.abs(b) + rms)))


def max_rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    rms = np.sqrt(np.mean(b * b)) if b.size else 0.0
    return float(np.max(np.abs(a - b) / (np.abs(b) + rms + 1e-300))) if b.size else 0.0
