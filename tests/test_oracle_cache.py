"""Pins of the oracle's two-cache layer: ring contents, chunked prefill and decode.

* the ring holds exactly the sinks plus the last R positions (the pages'
  description of the streaming cache, xllm-io review section 三), checked for
  every N up to 300 and against a hand-written table in tests/golden;
* the streaming cache size does not depend on the sequence length (constant
  memory, xllm-io review section 三 预填充阶段);
* chunked prefill equals one-shot attention for any chunk size, and prefill
  followed by decode steps equals one-shot attention at the last rows
  (paperlayer summary, section 2 Chunked Pre-filling).
"""
import os

import numpy as np
import pytest

import oracle
from duo_synth import rng, normal

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("S,R", [(16, 64), (2, 3), (0, 1), (4, 1), (0, 5)])
def test_ring_holds_sinks_and_last_recent(S, R):
    for N in range(0, 301):
        slots = oracle.ring_positions_after(N, S, R)
        held = sorted(p for p in slots if p >= 0)
        expect = sorted(set(range(min(S, N))) | set(range(max(S, N - R), N)))
        assert held == expect, (N, held, expect)
        assert len(slots) == S + R


def test_ring_matches_hand_table():
    rows = []
    with open(os.path.join(GOLDEN, "ring_s2_r3.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            rows.append([int(x) for x in line.split()])
    assert len(rows) == 11
    for row in rows:
        assert oracle.ring_positions_after(row[0], 2, 3) == row[1:], row


def test_ring_slot_closed_form():
    assert [oracle.ring_slot(p, 16, 64) for p in (0, 15, 16, 79, 80, 81, 143, 144)] == \
        [0, 15, 16, 79, 16, 17, 79, 16]


def _layer(mask, Hq, Hkv, D, scale, S, R, int4=False):
    return oracle.OracleLayer(Hq, Hkv, D, mask, scale, S, R, int4=int4)


@pytest.mark.parametrize("chunk", [1, 7, 64, 150])
def test_chunked_prefill_equals_one_shot(chunk):
    g = rng(21)
    T, Hq, Hkv, D, S, R = 150, 4, 2, 8, 3, 10
    q = normal(g, (T, Hq, D)).astype(np.float64)
    k, v = (normal(g, (T, Hkv, D)).astype(np.float64) for _ in range(2))
    mask = np.array([0, 1], np.uint8)
    ref = oracle.layer_attention(q, k, v, mask, 0.4, S, R)
    lay = _layer(mask, Hq, Hkv, D, 0.4, S, R)
    outs = []
    for a in range(0, T, chunk):
        outs.append(lay.prefill_chunk(q[a:a + chunk], k[a:a + chunk], v[a:a + chunk]))
    got = np.concatenate(outs)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    assert lay.n == T
    # constant memory: the ring never grows
    assert all(len(lay.ring[h]) == S + R for h in lay.ring)
    assert sorted(p for p in lay.ring_contents(0) if p >= 0) == \
        sorted(set(range(S)) | set(range(T - R, T)))


def test_prefill_then_decode_equals_one_shot():
    g = rng(22)
    T, steps, H, D, S, R = 100, 12, 3, 8, 4, 16
    q = normal(g, (T + steps, H, D)).astype(np.float64)
    k, v = (normal(g, (T + steps, H, D)).astype(np.float64) for _ in range(2))
    mask = np.array([1, 0, 0], np.uint8)
    ref = oracle.layer_attention(q, k, v, mask, 0.3, S, R)
    lay = _layer(mask, H, H, D, 0.3, S, R)
    lay.prefill_chunk(q[:T], k[:T], v[:T])
    for s in range(steps):
        o = lay.decode(q[T + s], k[T + s], v[T + s])
        np.testing.assert_allclose(o, ref[T + s], rtol=1e-12, atol=1e-13)


def test_append_then_decode_equals_one_shot():
    """Context filled without attention, then decode (the decode workloads)."""
    g = rng(23)
    N, steps, Hq, Hkv, D, S, R = 200, 5, 4, 2, 8, 16, 64
    q = normal(g, (N + steps, Hq, D)).astype(np.float64)
    k, v = (normal(g, (N + steps, Hkv, D)).astype(np.float64) for _ in range(2))
    mask = np.array([1, 0], np.uint8)
    ref = oracle.layer_attention(q, k, v, mask, 0.2, S, R)
    lay = _layer(mask, Hq, Hkv, D, 0.2, S, R)
    lay.append(k[:N], v[:N])
    for s in range(steps):
        np.testing.assert_allclose(lay.decode(q[N + s], k[N + s], v[N + s]), ref[N + s],
                                   rtol=1e-12, atol=1e-13)
    # each streaming decode query sees exactly S + R keys once N >= S + R
    held = [p for p in lay.ring_contents(1) if p >= 0]
    assert len(held) == S + R


def test_rows_subset_matches_full_chunk():
    g = rng(24)
    T, H, D = 64, 2, 4
    q, k, v = (normal(g, (T, H, D)).astype(np.float64) for _ in range(3))
    mask = np.array([1, 0], np.uint8)
    a = _layer(mask, H, H, D, 1.0, 2, 8).prefill_chunk(q, k, v)
    rows = [0, 5, 63]
    b = _layer(mask, H, H, D, 1.0, 2, 8).prefill_chunk(q, k, v, rows=rows)
    np.testing.assert_array_equal(a[rows], b[rows])
    assert np.isnan(b[1]).all()


def test_int4_layer_attends_over_dequantised_cache():
    """The int4 layer equals plain attention over the fma-dequantised K/V."""
    g = rng(25)
    T, Hq, Hkv, D = 40, 4, 2, 64
    q = normal(g, (T, Hq, D)).astype(np.float64)
    k, v = (normal(g, (T, Hkv, D)) for _ in range(2))
    mask = np.array([1, 0], np.uint8)
    lay = _layer(mask, Hq, Hkv, D, 0.125, 16, 64, int4=True)
    got = lay.prefill_chunk(q, k, v)
    kd, vd = k.astype(np.float64).copy(), v.astype(np.float64).copy()
    ck, sk, zk = oracle.quantize_int4_g32(k[:, 0])
    cv, sv, zv = oracle.quantize_int4_g32(v[:, 0])
    kd[:, 0] = oracle.dequantize_int4_g32(ck, sk, zk)
    vd[:, 0] = oracle.dequantize_int4_g32(cv, sv, zv)
    ref = oracle.layer_attention(q, kd, vd, mask, 0.125, 16, 64)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)
    # and the dequantised values are close to the originals
    assert np.abs(kd[:, 0] - k[:, 0]).max() < 0.5
