"""Host-side checks of the C ABI (no GPU): the library loads and exports every
symbol include/duo.h declares, buffer layouts, argument validation before any
HIP call, and the host helpers against the oracle bit for bit."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from duo_synth import rng

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from kv_cache_compression_duo_amd import _lib
    return _lib


def test_every_declared_symbol_is_exported():
    text = open(os.path.join(ROOT, "include", "duo.h")).read()
    names = set(re.findall(r"^[\w\s\*]*?\b(duo_\w+)\s*\(", text, flags=re.M))
    assert {"duo_append_kv", "duo_prefill_chunk", "duo_decode", "duo_mixed_forward"} <= names
    raw = ctypes.CDLL(_lib().LIB_PATH)
    missing = [n for n in sorted(names) if not hasattr(raw, n)]
    assert not missing, missing


def _desc(**kw):
    base = dict(n_q_heads=32, n_kv_heads=8, head_dim=128, n_retrieval_kv_heads=4, capacity=1000,
                softmax_scale=0.088)
    base.update(kw)
    return _lib().make_desc(**base)


def test_layout_sizes():
    L = _lib()
    lay = L.layout(_desc())
    # K and V arrays, then 32 readable rows (decode tiles start at any row)
    assert lay.retrieval_bytes == 2 * 4 * 1000 * 128 * 2 + 32 * 128 * 2
    assert lay.v_offset == 4 * 1000 * 128 * 2
    assert lay.streaming_bytes == 2 * 4 * 80 * 128 * 2
    lay4 = L.layout(_desc(kv_dtype="fp16", retrieval_dtype="int4", capacity=1024))
    codes = 4 * 1024 * 64
    sz = 4 * 1024 * 4 * 2 * 2
    assert lay4.v_offset == codes and lay4.k_sz_offset == 2 * codes
    assert lay4.v_sz_offset == 2 * codes + sz
    assert lay4.retrieval_bytes == 2 * codes + 2 * sz
    # 160 bytes per token per retrieval head for D = 128
    assert lay4.retrieval_bytes == 160 * 4 * 1024
    for x in (lay, lay4):
        for f in ("v_offset", "k_sz_offset", "v_sz_offset", "ring_v_offset"):
            assert getattr(x, f) % 256 == 0
    # no retrieval heads: no retrieval buffer
    assert L.layout(_desc(n_retrieval_kv_heads=0)).retrieval_bytes == 0


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=96), 2),
    (dict(n_q_heads=30), 1),
    (dict(n_q_heads=8 * 3), 2),          # group of 3
    (dict(n_retrieval_kv_heads=9), 1),
    (dict(recent=0), 1),
    (dict(sink=-1), 1),
    (dict(capacity=-5), 1),
    (dict(kv_dtype="bf16", retrieval_dtype="fp16"), 2),
    (dict(softmax_scale=float("inf")), 1),
    (dict(softmax_scale=0.0), 1),
    (dict(softmax_scale=-0.1), 1),
    # 4-bit cache: one head's code array must stay below 2^31 bytes
    (dict(kv_dtype="fp16", retrieval_dtype="int4", capacity=(1 << 25)), 2),
    # 16-bit cache: one head's rows plus 32 padding rows must stay below 2^31 bytes
    (dict(capacity=(1 << 23)), 2),
    # the batch and the KV heads are grid dimensions
    (dict(batch=65536), 2),
    (dict(n_q_heads=65536, n_kv_heads=65536, n_retrieval_kv_heads=4), 2),
    # sizes whose byte counts would not fit: 65535 x 65535 heads x 2^22 rows
    (dict(batch=65535, n_q_heads=65535, n_kv_heads=65535,
          n_retrieval_kv_heads=1, capacity=(1 << 22)), 4),
])
def test_bad_descriptor_rejected(kw, status):
    L = _lib()
    out = L.Layout()
    assert L.lib.duo_layer_layout(ctypes.byref(_desc(**kw)), ctypes.byref(out)) == status


def test_int4_capacity_limit():
    L = _lib()
    out = L.Layout()
    ok = _desc(kv_dtype="fp16", retrieval_dtype="int4", capacity=(1 << 25) - 32)
    assert L.lib.duo_layer_layout(ctypes.byref(ok), ctypes.byref(out)) == 0
    big = _desc(kv_dtype="fp16", retrieval_dtype="int4", capacity=(1 << 25) - 31)
    assert L.lib.duo_layer_layout(ctypes.byref(big), ctypes.byref(out)) == 2


@pytest.mark.parametrize("D", [64, 128])
def test_bf16_capacity_limit(D):
    L = _lib()
    out = L.Layout()
    last = (1 << 31) // (2 * D) - 32 - 1  # (cap + 32) * D * 2 < 2^31
    ok = _desc(head_dim=D, capacity=last, softmax_scale=D ** -0.5)
    assert L.lib.duo_layer_layout(ctypes.byref(ok), ctypes.byref(out)) == 0
    big = _desc(head_dim=D, capacity=last + 1, softmax_scale=D ** -0.5)
    assert L.lib.duo_layer_layout(ctypes.byref(big), ctypes.byref(out)) == 2


def test_init_validates_before_any_hip_call():
    L = _lib()
    h = ctypes.c_void_p()
    d = _desc()
    # null buffers
    assert L.lib.duo_layer_init(ctypes.byref(h), ctypes.byref(d), None, None, None, 0, None) == 1
    # misaligned buffers
    assert L.lib.duo_layer_init(ctypes.byref(h), ctypes.byref(d), 0x1008, 0x2000, 0x3000, 0,
                                None) == 3
    # existing tokens beyond capacity
    assert L.lib.duo_layer_init(ctypes.byref(h), ctypes.byref(d), 0x1000, 0x2000, 0x3000, 1001,
                                None) == 4
    assert L.lib.duo_layer_init(ctypes.byref(h), ctypes.byref(d), 0x1000, 0x2000, 0x3000, -1,
                                None) == 1
    assert h.value is None


def test_calls_reject_null_layer():
    L = _lib()
    assert L.lib.duo_append_kv(None, 0x1000, 0x1000, 1, None) == 1
    assert L.lib.duo_prefill_chunk(None, 0x1000, 0x1000, 0x1000, 1, 0x1000, None) == 1
    assert L.lib.duo_decode(None, 0x1000, 0x1000, 0x1000, 0x1000, None) == 1
    assert L.lib.duo_layer_tokens(None) == -1
    assert L.lib.duo_layer_destroy(None) == 0


def test_mixed_forward_validation():
    L = _lib()
    d = _desc()
    f = L.lib.duo_mixed_forward
    assert f(ctypes.byref(d), 0x1000, 0x1000, 0x1000, 0x1000, 0, 0x1000, None) == 1
    assert f(ctypes.byref(d), 0x1008, 0x1000, 0x1000, 0x1000, 16, 0x1000, None) == 3
    assert f(ctypes.byref(d), 0x1000, 0x1000, 0x1000, None, 16, 0x1000, None) == 1
    d16 = _desc(kv_dtype="fp16")
    assert f(ctypes.byref(d16), 0x1000, 0x1000, 0x1000, 0x1000, 16, 0x1000, None) == 2
    # a K tensor of 2^31 bytes (T * Hkv * D * 2) is beyond the kernel's 32-bit range
    big = (1 << 31) // (8 * 128 * 2)
    assert f(ctypes.byref(d), 0x1000, 0x1000, 0x1000, 0x1000, big, 0x1000, None) == 2


def test_mixed_alpha_grad_workspace_and_validation():
    L = _lib()
    f, ws = L.lib.duo_mixed_alpha_grad, L.lib.duo_mixed_alpha_grad_workspace
    d = _desc(n_q_heads=32, n_kv_heads=32, n_retrieval_kv_heads=0)
    # G = 1: one query head per block of 8 x 32 = 256 tokens; one fp32 partial per block
    assert ws(ctypes.byref(d), 16384) == 32 * 64 * 4
    assert ws(ctypes.byref(d), 257) == 32 * 2 * 4 + 0  # 256 B granularity: 256 already
    assert ws(ctypes.byref(d), 0) == 0
    dg = _desc()  # 32 q / 8 kv: G = 4, four query heads per block of 64 tokens
    assert ws(ctypes.byref(dg), 1000) == 256 * ((8 * 16 * 4 + 255) // 256)
    P, need = 0x1000, ws(ctypes.byref(d), 100)
    args = lambda **kw: [kw.get(n, dv) for n, dv in (  # noqa: E731
        ("q", P), ("k", P), ("v", P), ("dout", P), ("alpha", P), ("l1", 0.05), ("T", 100),
        ("grad", P), ("ws", P), ("ws_bytes", need))]
    # every case below fails validation before any HIP call
    assert f(ctypes.byref(d), *args(T=0), None) == 1
    assert f(ctypes.byref(d), *args(ws=None), None) == 1
    exact = 32 * 1 * 4  # T = 100: one 256-token tile per head (need rounds it up to 256 B)
    assert need >= exact
    assert f(ctypes.byref(d), *args(ws_bytes=exact - 4), None) == 1
    assert f(ctypes.byref(d), *args(grad=None), None) == 1
    assert f(ctypes.byref(d), *args(l1=float("inf")), None) == 1
    assert f(ctypes.byref(d), *args(ws=0x1004), None) == 3
    assert f(ctypes.byref(d), *args(dout=0x1008), None) == 3
    assert f(ctypes.byref(d), *args(grad=0x1002), None) == 3
    d16 = _desc(n_q_heads=32, n_kv_heads=32, n_retrieval_kv_heads=0, kv_dtype="fp16")
    assert f(ctypes.byref(d16), *args(), None) == 2
    big = (1 << 31) // (32 * 128 * 2)
    assert f(ctypes.byref(d), *args(T=big, ws_bytes=1 << 40), None) == 2


def test_binarize_gates_matches_oracle_bit_for_bit():
    from kv_cache_compression_duo_amd import binarize_gates
    g = rng(52)
    for _ in range(300):
        n = int(g.integers(1, 300))
        a = g.uniform(-0.2, 1.2, n).astype(np.float32)
        if n > 3 and g.integers(0, 2):
            a[: n // 3] = a[0]  # ties
        s = float(g.choice([0.0, 1.0, g.uniform(0.0, 1.0), 0.29, 0.5]))
        assert binarize_gates(a, s) == oracle.binarize_gates(a.astype(np.float64), s).tolist()
    L = _lib()
    a = (ctypes.c_float * 3)(0.1, float("nan"), 0.3)
    m = (ctypes.c_uint8 * 3)()
    assert L.lib.duo_binarize_gates(a, 3, 0.5, m) == 1
    b = (ctypes.c_float * 3)(0.1, 0.2, 0.3)
    assert L.lib.duo_binarize_gates(b, 3, -0.1, m) == 1
    assert L.lib.duo_binarize_gates(b, 3, 1.5, m) == 1
    assert L.lib.duo_binarize_gates(b, 0, 0.5, m) == 1


def test_reorder_head_rows_matches_oracle_bit_for_bit():
    from kv_cache_compression_duo_amd import reorder_head_rows
    g = rng(53)
    for dtype in (np.float32, np.uint16, np.float64):
        n, rph, cols = 6, 4, 10
        w = (g.standard_normal((n * rph, cols)) * 1000).astype(dtype)
        perm = g.permutation(n)
        np.testing.assert_array_equal(reorder_head_rows(w, perm, rph),
                                      oracle.reorder_head_rows(w, perm, rph))
    L = _lib()
    src = np.arange(12, dtype=np.float32)
    dst = np.zeros(12, np.float32)
    bad = (ctypes.c_int32 * 3)(0, 0, 2)  # not a permutation
    assert L.lib.duo_reorder_head_rows(src.ctypes.data, dst.ctypes.data, bad, 3, 1, 16) == 1
    ok = (ctypes.c_int32 * 3)(2, 0, 1)
    assert L.lib.duo_reorder_head_rows(src.ctypes.data, src.ctypes.data, ok, 3, 1, 16) == 3
    assert L.lib.duo_reorder_head_rows(src.ctypes.data, dst.ctypes.data, ok, 3, 1, 16) == 0
    np.testing.assert_array_equal(dst, np.concatenate([src[8:12], src[0:4], src[4:8]]))


def test_ragged_init_and_sequence_calls_validate_first():
    L = _lib()
    h = ctypes.c_void_p()
    d = _desc(batch=3)  # capacity 1000
    init = L.lib.duo_layer_init_ragged
    by = ctypes.byref
    assert init(by(h), by(d), 0x1000, 0x2000, 0x3000, None, None) == 1
    assert init(by(h), by(d), 0x1000, 0x2000, 0x3000, (ctypes.c_int64 * 3)(10, -1, 7), None) == 1
    assert init(by(h), by(d), 0x1000, 0x2000, 0x3000, (ctypes.c_int64 * 3)(10, 5, 1001),
                None) == 4
    assert init(by(h), by(d), 0x1008, 0x2000, 0x3000, (ctypes.c_int64 * 3)(10, 5, 7), None) == 3
    assert h.value is None
    assert L.lib.duo_layer_sequence_tokens(None, 0) == -1
    assert L.lib.duo_append_kv_seq(None, 0, 0x1000, 0x1000, 4, None) == 1
    assert L.lib.duo_prefill_chunk_seq(None, 0, 0x1000, 0x1000, 0x1000, 4, 0x1000, None) == 1


def test_status_strings():
    L = _lib()
    assert L.status_string(0) == "ok"
    assert "capacity" in L.status_string(4)


def test_head_permutation_matches_oracle():
    from kv_cache_compression_duo_amd import head_permutation
    g = rng(51)
    for _ in range(200):
        H = int(g.integers(1, 65))
        mask = [int(x) for x in g.integers(0, 2, size=H)]
        assert head_permutation(mask) == oracle.head_permutation(mask)
    assert head_permutation([1, 0, 0, 0, 0, 1, 0, 0]) == ([0, 5, 1, 2, 3, 4, 6, 7], 2)


def test_ring_slot_matches_oracle():
    from kv_cache_compression_duo_amd import ring_slot
    for S, R in [(16, 64), (2, 3), (0, 1), (5, 7)]:
        for p in range(0, 500):
            assert ring_slot(p, S, R) == oracle.ring_slot(p, S, R)
    assert ring_slot(-1, 16, 64) == -1
    assert ring_slot(3, 16, 0) == -1


def test_binding_has_no_host_path():
    """The Python calls refuse host tensors and a host device before any
    library call: there is no CPU fallback."""
    import torch
    import kv_cache_compression_duo_amd as duo
    q = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16)
    a = torch.zeros(2)
    with pytest.raises(ValueError, match="not a GPU"):
        duo.mixed_forward(q, q, q, a, softmax_scale=0.125)
    with pytest.raises(ValueError, match="not a GPU"):
        duo.mixed_alpha_grad(q, q, q, q, a, softmax_scale=0.125)
    with pytest.raises(ValueError, match="not a GPU"):
        duo.DuoLayer(n_q_heads=2, n_kv_heads=2, head_dim=64, n_retrieval_kv_heads=1,
                     capacity=16, softmax_scale=0.125, device="cpu")


def test_one_hip_runtime_whatever_the_import_order():
    """Importing the package before torch must not load a second HIP runtime:
    the library has to share torch's, which owns the device memory and streams
    it is handed (a second runtime in the process sees no device)."""
    import ast
    import subprocess
    import sys
    code = ("import kv_cache_compression_duo_amd, torch\n"
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         timeout=300, check=True).stdout
    paths = ast.literal_eval(out.strip().splitlines()[-1])
    assert len(paths) == 1, paths
