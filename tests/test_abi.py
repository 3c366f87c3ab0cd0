"""The C ABI on the host: the library loads, exports every function the header
declares, and rejects bad arguments before anything is enqueued (no GPU)."""
import ctypes
import os
import re

import pytest

import evs_synth as es
from attention_dna_lms_amd import evs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "evs.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(evs_[a-z_]+)\s*\(", src)))


def test_header_declares_the_hot_path():
    names = _declared()
    for n in ("evs_prefill", "evs_block_verify", "evs_rollback", "evs_verify_sample"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = evs.lib()
    for n in _declared():
        assert hasattr(L, n), n
    assert set(_declared()) == set(evs.EXPORTS)


def test_status_strings():
    assert evs.status_string(0) == "ok"
    assert evs.status_string(-3) == "call out of order"


def _desc(cfg):
    return evs.model_desc(cfg)


def test_weights_bytes_and_canonical_shapes():
    L = evs.lib()
    cfg = es.stack_7b()
    d = _desc(cfg)
    n = ctypes.c_size_t()
    assert L.evs_weights_bytes(ctypes.byref(d), ctypes.byref(n)) == 0
    # packed matrices are exactly the canonical bytes (no padding: every size is a tile multiple
    # and every K a multiple of 8 k-steps, one range per wave)
    assert n.value >= cfg.weight_bytes()
    assert n.value - cfg.weight_bytes() < 64 * 1024 * 1024
    cnt = ctypes.c_int32()
    assert L.evs_canonical_count(ctypes.byref(d), ctypes.byref(cnt)) == 0
    names = evs.canonical_order(cfg)
    assert cnt.value == len(names) == len(es.weight_names(cfg))
    for i, (name, shape) in enumerate(es.weight_names(cfg)):
        r, c, dt = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
        assert L.evs_canonical_shape(ctypes.byref(d), i, ctypes.byref(r), ctypes.byref(c), ctypes.byref(dt)) == 0
        assert names[i] == name and (r.value, c.value) == shape
        f32_param = name.endswith((".taps", ".lam", ".res"))
        assert dt.value == (evs.EVS_F32 if f32_param else evs.EVS_BF16)


@pytest.mark.parametrize("mutate", [
    lambda c: setattr(c, "d_model", 100),                 # not a multiple of 32
    lambda c: setattr(c, "vocab", 1),
    lambda c: c.blocks.__setitem__(0, es.Block("iir", iir_states=17)),
    lambda c: c.blocks.__setitem__(0, es.Block("attn", n_heads=3, head_dim=32)),   # 96 != d
    lambda c: c.blocks.__setitem__(0, es.Block("mlp", d_ff=100)),
    lambda c: c.blocks.__setitem__(0, es.Block("fir", fir_len=0)),
])
def test_bad_descriptors_rejected(mutate):
    cfg = es.small_stack()
    mutate(cfg)
    d = _desc(cfg)
    n = ctypes.c_size_t()
    assert evs.lib().evs_weights_bytes(ctypes.byref(d), ctypes.byref(n)) == -1


def test_model_create_and_state_sizes_without_device_access():
    L = evs.lib()
    cfg = es.stack_7b()
    d = _desc(cfg)
    fake = ctypes.c_void_p(0x100000)          # never dereferenced by create
    h = ctypes.c_void_p()
    assert L.evs_model_create(ctypes.byref(d), fake, ctypes.byref(h)) == 0
    assert L.evs_model_create(ctypes.byref(d), ctypes.c_void_p(0x100001), ctypes.byref(ctypes.c_void_p())) == -1
    sb, wb = ctypes.c_size_t(), ctypes.c_size_t()
    assert L.evs_state_bytes(h, 1, 8192 + 1024, 13, ctypes.byref(sb), ctypes.byref(wb)) == 0
    # KV: 4 attention layers x (K + V) x cap x 4096 x 2 bytes dominates the state
    kv = 4 * 2 * (8192 + 1024) * 4096 * 2
    # plus FIR rings (9 x 4 MB + 10 x 0.5 MB) and IIR position buffers (9 x 6.8 MB)
    assert kv + 90e6 <= sb.value < kv + 128 * 1024 * 1024
    assert wb.value < 64 * 1024 * 1024
    assert L.evs_state_bytes(h, 1, 8192, 0, ctypes.byref(sb), ctypes.byref(wb)) == -1
    assert L.evs_state_bytes(h, 1, 8192, 145, ctypes.byref(sb), ctypes.byref(wb)) == -1
    assert L.evs_state_bytes(h, 64, 8192, 100, ctypes.byref(sb), ctypes.byref(wb)) == -2
    L.evs_model_destroy(h)


def test_verify_sample_rejects_bad_arguments_before_launch():
    L = evs.lib()
    p = ctypes.c_void_p(0x1000)
    z = ctypes.c_void_p(0)
    # batch 0, bad kind, greedy=0 without uniforms, temperature 0, too-large block
    assert L.evs_verify_sample(0, 4, 512, p, 1, p, p, p, 1.0, 0, 0, p, p, z, z, z) == -1
    assert L.evs_verify_sample(1, 4, 512, p, 9, p, p, p, 1.0, 0, 0, p, p, z, z, z) == -1
    assert L.evs_verify_sample(1, 4, 512, p, 1, p, p, z, 1.0, 0, 0, p, p, z, z, z) == -1
    assert L.evs_verify_sample(1, 4, 512, p, 1, p, p, p, 0.0, 0, 0, p, p, z, z, z) == -1
    assert L.evs_verify_sample(1, 40, 512, p, 1, p, p, p, 1.0, 0, 0, p, p, z, z, z) == -5
    assert L.evs_verify_sample(1, 64, 4, p, 1, p, p, p, 1.0, 0, 0, p, p, z, z, z) == -1


@pytest.mark.parametrize("mode", [[], ["--c5"], ["--soak", "64"], ["--stream-floor"]])
def test_bench_refuses_more_than_one_gpu(mode):
    """bench.py measures one GPU: any mode with --gpus N > 1 exits with status 2
    and says so, before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"] + mode,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
