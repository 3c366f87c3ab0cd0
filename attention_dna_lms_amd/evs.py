"""Python binding of libevs (include/evs.h): ctypes marshalling.

Every function named evs_* here forwards to the C function of the same name;
tensors are passed as device pointers and the current torch stream as the HIP
stream. ``Model`` and ``State`` own the device buffers (torch tensors) that
the C API asks the caller for. ``generate`` / ``generate_native`` (model
card, "Library") only allocate the buffers, draw the uniforms the caller did
not pass from a seeded device generator, and call evs_prefill and
evs_generate; every step of the method runs in the library. There is no
fallback: if libevs.so is missing or cannot be loaded, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_uint64, c_void_p

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libevs.so")

EVS_FIR, EVS_IIR, EVS_ATTN, EVS_MLP = 1, 2, 3, 4
EVS_BF16, EVS_F32, EVS_I32, EVS_BF16_FP8W = 1, 2, 3, 4
EVS_TARGET_LOGITS_BF16, EVS_TARGET_LOGITS_F32, EVS_TARGET_PROBS_F32 = 1, 2, 3
EVS_ST_T, EVS_ST_IIR_BUF, EVS_ST_IIR_SLOT, EVS_ST_FIR_RING, EVS_ST_IIR, EVS_ST_K, EVS_ST_VT, EVS_ST_ERROR = range(1, 9)
EVS_ERR_TOKEN, EVS_ERR_CONTEXT, EVS_ERR_NKEEP, EVS_ERR_DRAFT, EVS_ERR_INDEX = 1, 2, 4, 8, 16
STATUS = {0: "EVS_OK", -1: "EVS_E_INVALID", -2: "EVS_E_RANGE", -3: "EVS_E_STATE", -4: "EVS_E_HIP",
          -5: "EVS_E_UNSUPPORTED"}
_KINDS = {"fir": EVS_FIR, "iir": EVS_IIR, "attn": EVS_ATTN, "mlp": EVS_MLP}
_TORCH_DT = {EVS_BF16: torch.bfloat16, EVS_F32: torch.float32, EVS_I32: torch.int32}

# exported symbols declared in include/evs.h
EXPORTS = ("evs_status_string", "evs_canonical_count", "evs_canonical_shape", "evs_weights_bytes",
           "evs_model_create", "evs_pack_weights", "evs_model_destroy", "evs_state_bytes", "evs_state_create",
           "evs_state_destroy", "evs_state_tensor", "evs_state_error", "evs_prefill", "evs_block_verify",
           "evs_rollback", "evs_verify_sample", "evs_state_export", "evs_draft", "evs_state_timing",
           "evs_state_timing_read", "evs_block_verify_noalloc", "evs_generate_workspace_bytes", "evs_generate",
           "evs_measure_weight_stream")
EVS_W_IN, EVS_W_OUT, EVS_W_GU, EVS_W_DOWN, EVS_W_LM = 1, 2, 3, 4, 5
EVS_DRAFT_NONE, EVS_DRAFT_MODEL, EVS_DRAFT_TABLE = 0, 1, 2
EVS_NOALLOC_SCRATCH_BYTES = 32 << 20
EVS_KC_GEMM, EVS_KC_ATTN = 1, 2


class EvsError(RuntimeError):
    def __init__(self, status, where):
        super().__init__(f"{where}: {STATUS.get(status, status)}")
        self.status = status


class BlockDesc(ctypes.Structure):
    _fields_ = [("kind", c_int32), ("fir_len", c_int32), ("iir_states", c_int32), ("n_heads", c_int32),
                ("head_dim", c_int32), ("d_ff", c_int32)]


class ModelDesc(ctypes.Structure):
    _fields_ = [("d_model", c_int32), ("vocab", c_int32), ("n_blocks", c_int32), ("dtype", c_int32),
                ("norm_eps", c_float), ("blocks", POINTER(BlockDesc)), ("inject_dim", c_int32),
                ("max_slots", c_int32)]


class DraftSource(ctypes.Structure):
    _fields_ = [("source", c_int32), ("drafter", c_void_p), ("drafter_state", c_void_p), ("table_dev", c_void_p),
                ("table_len", c_int32), ("replace_dev", c_void_p)]


class GenParams(ctypes.Structure):
    _fields_ = [("n_tokens", c_int32), ("gamma", c_int32), ("greedy", c_int32), ("temperature", c_float),
                ("top_k", c_int32), ("rounds_cap", c_int32), ("u_first_dev", c_void_p), ("u_target_dev", c_void_p),
                ("u_draft_dev", c_void_p)]


class TensorDesc(ctypes.Structure):
    _fields_ = [("offset", c_uint64), ("dtype", c_int32), ("ndim", c_int32), ("shape", c_int64 * 6),
                ("strides", c_int64 * 6)]


_lib = None


def lib():
    """The loaded libevs.so (raises if it is absent or fails to load)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libevs.so not built ({LIB_PATH}); run python -m attention_dna_lms_amd.build")
    L = ctypes.CDLL(LIB_PATH)
    L.evs_status_string.restype = ctypes.c_char_p
    L.evs_status_string.argtypes = [c_int32]
    sig = {
        "evs_canonical_count": [POINTER(ModelDesc), POINTER(c_int32)],
        "evs_canonical_shape": [POINTER(ModelDesc), c_int32, POINTER(c_int64), POINTER(c_int64), POINTER(c_int32)],
        "evs_weights_bytes": [POINTER(ModelDesc), POINTER(c_size_t)],
        "evs_model_create": [POINTER(ModelDesc), c_void_p, POINTER(c_void_p)],
        "evs_pack_weights": [c_void_p, POINTER(c_void_p), c_void_p],
        "evs_state_bytes": [c_void_p, c_int32, c_int32, c_int32, POINTER(c_size_t), POINTER(c_size_t)],
        "evs_state_create": [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, POINTER(c_void_p)],
        "evs_state_tensor": [c_void_p, c_int32, c_int32, POINTER(TensorDesc)],
        "evs_state_error": [c_void_p, POINTER(c_int32), c_int32, c_void_p],
        "evs_prefill": [c_void_p, c_void_p, c_void_p, POINTER(c_int32), c_void_p, c_void_p],
        "evs_block_verify": [c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p],
        "evs_block_verify_noalloc": [c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p],
        "evs_rollback": [c_void_p, c_void_p, c_void_p],
        "evs_state_timing": [c_void_p, c_int32, c_int64],
        "evs_state_timing_read": [c_void_p, c_int32, POINTER(ctypes.c_double), POINTER(c_int64),
                                  POINTER(ctypes.c_double), c_void_p],
        "evs_verify_sample": [c_int32, c_int32, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_float,
                              c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p],
        "evs_state_export": [c_void_p, c_int32, c_void_p],
        "evs_measure_weight_stream": [c_void_p, c_int32, c_int32, c_void_p, c_size_t, POINTER(ctypes.c_double),
                                      c_void_p],
        "evs_generate_workspace_bytes": [c_void_p, c_void_p, POINTER(GenParams), POINTER(DraftSource),
                                         POINTER(c_size_t)],
        "evs_generate": [c_void_p, c_void_p, c_void_p, POINTER(GenParams), POINTER(DraftSource), c_void_p, c_void_p,
                         c_void_p, POINTER(c_int32), c_void_p],
        "evs_draft": [c_void_p, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_void_p,
                      c_float, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.restype = c_int32
        f.argtypes = args
    L.evs_model_destroy.argtypes = [c_void_p]
    L.evs_model_destroy.restype = None
    L.evs_state_destroy.argtypes = [c_void_p]
    L.evs_state_destroy.restype = None
    _lib = L
    return L


def _check(st, where):
    if st != 0:
        raise EvsError(st, where)


def _ptr(t):
    return c_void_p(0 if t is None else t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream)


def _aligned_buffer(nbytes, device):
    """uint8 device buffer of nbytes whose data pointer is 256-byte aligned."""
    raw = torch.empty(max(int(nbytes), 1) + 256, dtype=torch.uint8, device=device)
    off = (-raw.data_ptr()) % 256
    return raw, raw[off: off + max(int(nbytes), 1)]


def model_desc(cfg, fp8_weights=False):
    """ModelDesc from a config with d_model, vocab, dtype ('bf16'|'f32'),
    norm_eps and blocks (kind, fir_len, iir_states, n_heads, head_dim, d_ff);
    fp8_weights selects EVS_BF16_FP8W for a bf16 config."""
    blocks = (BlockDesc * max(len(cfg.blocks), 1))()
    for i, b in enumerate(cfg.blocks):
        blocks[i] = BlockDesc(_KINDS[b.kind], b.fir_len, b.iir_states, b.n_heads, b.head_dim, b.d_ff)
    if fp8_weights and cfg.dtype != "bf16":
        raise ValueError("FP8 weights are a variant of bf16 models")
    dt = EVS_BF16_FP8W if fp8_weights else (EVS_BF16 if cfg.dtype == "bf16" else EVS_F32)
    d = ModelDesc(cfg.d_model, cfg.vocab, len(cfg.blocks), dt, float(cfg.norm_eps), blocks,
                  int(getattr(cfg, "inject_dim", 0)), int(getattr(cfg, "max_slots", 0)))
    d._keep = blocks
    return d


def canonical_order(cfg):
    """Names of the canonical tensors in evs_pack_weights order."""
    names = ["embed"]
    for i, b in enumerate(cfg.blocks):
        if b.kind == "fir":
            names += [f"b{i}.w_in", f"b{i}.taps", f"b{i}.w_out"]
        elif b.kind == "iir":
            names += [f"b{i}.w_in", f"b{i}.lam", f"b{i}.res", f"b{i}.w_out"]
        elif b.kind == "attn":
            names += [f"b{i}.w_in", f"b{i}.w_out"]
        else:
            names += [f"b{i}.w_gu", f"b{i}.w_down"]
    names.append("lm_head")
    if getattr(cfg, "inject_dim", 0):
        names += ["inject", "pos", "markov"]
    return names


class Model:
    """A packed model on the device (evs_model_create + evs_pack_weights); with
    fp8_weights the block projections are quantised to FP8 E4M3 at packing."""

    def __init__(self, cfg, weights, device="cuda", fp8_weights=False):
        L = lib()
        self.cfg = cfg
        self.fp8_weights = fp8_weights
        self.desc = model_desc(cfg, fp8_weights)
        n = c_size_t()
        _check(L.evs_weights_bytes(ctypes.byref(self.desc), ctypes.byref(n)), "evs_weights_bytes")
        self._raw, self.packed = _aligned_buffer(n.value, device)
        h = c_void_p()
        _check(L.evs_model_create(ctypes.byref(self.desc), _ptr(self.packed), ctypes.byref(h)), "evs_model_create")
        self.handle = h
        cnt = c_int32()
        _check(L.evs_canonical_count(ctypes.byref(self.desc), ctypes.byref(cnt)), "evs_canonical_count")
        names = canonical_order(cfg)
        assert len(names) == cnt.value
        tens = []
        for i, name in enumerate(names):
            r, c, dt = c_int64(), c_int64(), c_int32()
            _check(L.evs_canonical_shape(ctypes.byref(self.desc), i, ctypes.byref(r), ctypes.byref(c),
                                         ctypes.byref(dt)), "evs_canonical_shape")
            t = weights[name].to(device=device, dtype=_TORCH_DT[dt.value]).contiguous()
            if tuple(t.shape) != (r.value, c.value):
                raise ValueError(f"{name}: shape {tuple(t.shape)} != {(r.value, c.value)}")
            tens.append(t)
        ptrs = (c_void_p * len(tens))(*[t.data_ptr() for t in tens])
        _check(L.evs_pack_weights(self.handle, ptrs, _stream()), "evs_pack_weights")
        torch.cuda.current_stream().synchronize()
        del tens

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.evs_model_destroy(self.handle)
            self.handle = None


class State:
    """Inference state of `batch` sequences plus the call workspace."""

    def __init__(self, model: Model, batch: int, max_ctx: int, max_block: int, device="cuda", workspace=True):
        """workspace=False: no workspace of its own (evs_block_verify_noalloc only)."""
        L = lib()
        self.model = model
        self.B, self.max_ctx, self.max_block = batch, max_ctx, max_block
        sb, wb = c_size_t(), c_size_t()
        _check(L.evs_state_bytes(model.handle, batch, max_ctx, max_block, ctypes.byref(sb), ctypes.byref(wb)),
               "evs_state_bytes")
        self.state_bytes, self.workspace_bytes = sb.value, wb.value
        self._sraw, self.buf = _aligned_buffer(sb.value, device)
        self._wraw, self.ws = _aligned_buffer(wb.value, device) if workspace else (None, None)
        h = c_void_p()
        _check(L.evs_state_create(model.handle, batch, max_ctx, max_block, _ptr(self.buf), _ptr(self.ws), _stream(),
                                  ctypes.byref(h)), "evs_state_create")
        self.handle = h

    def tensor(self, what: int, block: int = -1) -> torch.Tensor:
        """A torch view of a state tensor (evs_state_tensor)."""
        d = TensorDesc()
        _check(lib().evs_state_tensor(self.handle, what, block, ctypes.byref(d)), "evs_state_tensor")
        dt = _TORCH_DT[d.dtype]
        es = torch.tensor([], dtype=dt).element_size()
        shape = [d.shape[i] for i in range(d.ndim)]
        strides = [d.strides[i] for i in range(d.ndim)]
        n = 1
        for s in shape:
            n *= s
        flat = self.buf[d.offset: d.offset + n * es].view(dt)
        return torch.as_strided(flat, shape, strides)

    def error(self, clear: bool = False) -> int:
        w = c_int32()
        _check(lib().evs_state_error(self.handle, ctypes.byref(w), int(clear), _stream()), "evs_state_error")
        return w.value

    def timing(self, enable: bool, context_hint: int = 0):
        """Enable or disable per-launch event timing (evs_state_timing)."""
        _check(lib().evs_state_timing(self.handle, int(enable), int(context_hint)), "evs_state_timing")

    def timing_read(self, kernel_class: int):
        """(total ms, launches, algorithmic bytes) of the recorded launches of a class."""
        ms, n, by = ctypes.c_double(), c_int64(), ctypes.c_double()
        _check(lib().evs_state_timing_read(self.handle, int(kernel_class), ctypes.byref(ms), ctypes.byref(n),
                                           ctypes.byref(by), _stream()), "evs_state_timing_read")
        return ms.value, n.value, by.value

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.evs_state_destroy(self.handle)
            self.handle = None


# ------------------------------------------------------------------ hot path
def evs_prefill(model: Model, state: State, tokens: torch.Tensor, seq_offsets, last_logits=None):
    offs = (c_int32 * len(seq_offsets))(*[int(x) for x in seq_offsets])
    _check(lib().evs_prefill(model.handle, state.handle, _ptr(tokens), offs, _ptr(last_logits), _stream()),
           "evs_prefill")


def evs_block_verify(model: Model, state: State, cand: torch.Tensor, gamma: int, logits: torch.Tensor):
    _check(lib().evs_block_verify(model.handle, state.handle, _ptr(cand), int(gamma), _ptr(logits), _stream()),
           "evs_block_verify")


def evs_block_verify_noalloc(model: Model, state: State, cand: torch.Tensor, gamma: int, logits: torch.Tensor):
    _check(lib().evs_block_verify_noalloc(model.handle, state.handle, _ptr(cand), int(gamma), _ptr(logits),
                                          _stream()), "evs_block_verify_noalloc")


def evs_rollback(state: State, n_keep=None):
    _check(lib().evs_rollback(state.handle, _ptr(n_keep), _stream()), "evs_rollback")


def evs_verify_sample(batch, gamma, vocab, target, target_kind, q, draft, u, temperature, top_k, greedy,
                      n_accepted, next_token, n_keep=None, error=None):
    _check(lib().evs_verify_sample(int(batch), int(gamma), int(vocab), _ptr(target), int(target_kind), _ptr(q),
                                   _ptr(draft), _ptr(u), float(temperature), int(top_k), int(greedy),
                                   _ptr(n_accepted), _ptr(next_token), _ptr(n_keep), _ptr(error), _stream()),
           "evs_verify_sample")


def evs_state_export(state: State, block: int, dst=None):
    """Export the residual rows after `block` during evs_block_verify into dst
    (f32 [B, max_block, d]); block -1 turns the export off."""
    _check(lib().evs_state_export(state.handle, int(block), _ptr(dst)), "evs_state_export")


def evs_draft(drafter: Model, dstate: State, batch, hidden, hidden_rows, hidden_index, last, gamma, u,
              temperature, top_k, greedy, logits, drafts, q=None):
    _check(lib().evs_draft(drafter.handle, dstate.handle, int(batch), _ptr(hidden), int(hidden_rows),
                           _ptr(hidden_index), _ptr(last), int(gamma), _ptr(u), float(temperature), int(top_k),
                           int(greedy), _ptr(logits), _ptr(drafts), _ptr(q), _stream()), "evs_draft")


def _gen_structs(n_tokens, gamma, greedy, temperature, top_k, rounds_cap, u_first, u_target, u_draft, source,
                 drafter=None, drafter_state=None, table=None, replace=None):
    p = GenParams(int(n_tokens), int(gamma), int(bool(greedy)), float(temperature), int(top_k), int(rounds_cap),
                  _ptr(u_first), _ptr(u_target), _ptr(u_draft))
    d = DraftSource(int(source), drafter.handle if drafter is not None else None,
                    drafter_state.handle if drafter_state is not None else None, _ptr(table),
                    0 if table is None else int(table.shape[-1]), _ptr(replace))
    return p, d


def evs_generate_workspace_bytes(model: Model, state: State, params: GenParams, source: DraftSource) -> int:
    n = c_size_t()
    _check(lib().evs_generate_workspace_bytes(model.handle, state.handle, ctypes.byref(params), ctypes.byref(source),
                                              ctypes.byref(n)), "evs_generate_workspace_bytes")
    return n.value


def evs_generate(model: Model, state: State, last_logits, params: GenParams, source: DraftSource, work, ids,
                 stats) -> int:
    """Returns the number of rounds."""
    n = c_int32()
    _check(lib().evs_generate(model.handle, state.handle, _ptr(last_logits), ctypes.byref(params),
                              ctypes.byref(source), _ptr(work), _ptr(ids), _ptr(stats), ctypes.byref(n), _stream()),
           "evs_generate")
    return n.value


class GenResult:
    """ids [B, n_tokens] (int64 numpy), tok_s (generated tokens per second,
    all sequences, from the first draw to the last round), mean_tau (mean
    tokens emitted per round, before the cut at n_tokens), rounds."""

    def __init__(self, ids, tok_s, mean_tau, rounds, stats):
        self.ids, self.tok_s, self.mean_tau, self.rounds, self.stats = ids, tok_s, mean_tau, rounds, stats


def generate(model: Model, state: State, prompts, n_tokens, gamma=12, greedy=False, temperature=1.0, top_k=4,
             drafter: Model = None, drafter_state: State = None, export_block=None, table=None, replace=None,
             u_first=None, u_target=None, u_draft=None, rounds_cap=None, seed=0):
    """Prompts (list of int arrays, one per sequence of `state`) -> GenResult,
    through evs_prefill and evs_generate (model card, "Library": generate).
    Drafts from `drafter` (with `drafter_state`, reading the target's
    residual rows after block `export_block`), or from `table` [B, L]
    (+ `replace`), or none (gamma must then be 0: generate_native).
    Uniforms are taken as given, or drawn on the device from `seed`."""
    dev = state.buf.device
    B = state.B
    if len(prompts) != B:
        raise ValueError("one prompt per sequence of the state")
    rounds_cap = int(rounds_cap or n_tokens)
    src = EVS_DRAFT_MODEL if drafter is not None else EVS_DRAFT_TABLE if table is not None else EVS_DRAFT_NONE
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))

    def uni(x, shape):
        return torch.as_tensor(x, dtype=torch.float32, device=dev).contiguous() if x is not None else \
            torch.rand(shape, generator=g, device=dev, dtype=torch.float32)
    uf = uni(u_first, (B,))
    ut = uni(u_target, (rounds_cap, B, gamma + 1))
    ud = uni(u_draft, (rounds_cap, B, max(gamma, 1))) if src == EVS_DRAFT_MODEL else None
    tab = None if table is None else torch.as_tensor(table, dtype=torch.int32, device=dev).contiguous()
    rep = None if replace is None else torch.as_tensor(replace, dtype=torch.int32, device=dev).contiguous()
    p, d = _gen_structs(n_tokens, gamma, greedy, temperature, top_k, rounds_cap, uf, ut, ud, src, drafter,
                        drafter_state, tab, rep)
    hidden = None
    if src == EVS_DRAFT_MODEL:
        hidden = torch.zeros(B * state.max_block * model.cfg.d_model, dtype=torch.float32, device=dev)
        evs_state_export(state, export_block, hidden)
    flat = torch.as_tensor(np.concatenate([np.asarray(x, np.int32) for x in prompts]), device=dev)
    offs = np.concatenate([[0], np.cumsum([len(x) for x in prompts])])
    last = torch.zeros(B, model.cfg.vocab, dtype=_TORCH_DT[model.desc.dtype if model.desc.dtype != EVS_BF16_FP8W
                                                           else EVS_BF16], device=dev)
    evs_prefill(model, state, flat, offs, last)
    work = _aligned_buffer(evs_generate_workspace_bytes(model, state, p, d), dev)[1]
    ids = torch.zeros(B, n_tokens, dtype=torch.int32, device=dev)
    stats = torch.zeros(B, 2, dtype=torch.int32, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    try:
        rounds = evs_generate(model, state, last, p, d, work, ids, stats)
    finally:
        if hidden is not None:
            evs_state_export(state, -1)
    e1.record()
    torch.cuda.synchronize()
    st = stats.cpu().numpy()
    tok_s = B * n_tokens / (e0.elapsed_time(e1) / 1e3)
    mean_tau = float(st[:, 1].sum() / max(st[:, 0].sum(), 1))
    return GenResult(ids.cpu().numpy().astype(np.int64), tok_s, mean_tau, rounds, st)


def generate_native(model: Model, state: State, prompts, n_tokens, greedy=False, **kw):
    """Native decoding (one token per target step) through the same loop."""
    return generate(model, state, prompts, n_tokens, gamma=0, greedy=greedy, **kw)


def evs_measure_weight_stream(model: Model, block: int, which: int, sink) -> float:
    """Enqueue the weight stream of one projection (measurement aid); returns its bytes."""
    by = ctypes.c_double()
    _check(lib().evs_measure_weight_stream(model.handle, int(block), int(which), _ptr(sink),
                                           sink.numel() * sink.element_size(), ctypes.byref(by), _stream()),
           "evs_measure_weight_stream")
    return by.value


def status_string(status: int) -> str:
    return lib().evs_status_string(int(status)).decode()
