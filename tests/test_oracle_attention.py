"""Pins of the oracle's attention against things other than itself.

* pure-Python brute force (math.exp, explicit key sets) on tiny inputs;
* a library routine: torch's scaled_dot_product_attention in float64 on the
  CPU with a boolean mask;
* closed forms (single token, zero query, planted key, window of one);
* the pages' invariants: alpha = 1 is full attention, alpha = 0 is streaming
  attention (xllm-io review, section 三 整体框架 / 核心公式), a window that
  covers the whole sequence makes streaming equal full, and the all-streaming
  layer is the StreamingLLM special case.
"""
import math

import numpy as np
import pytest

import oracle
from duo_synth import rng, normal


def _brute(q, k, v, q_pos, k_pos, scale, kind, S, R):
    """Straight from the definition, one query and one key at a time."""
    Tq, D = len(q), len(q[0])
    out = []
    for a in range(Tq):
        i = int(q_pos[a])
        keys = []
        for b in range(len(k)):
            j = int(k_pos[b])
            if j > i:
                continue
            if kind == "streaming":
                sinks = set(range(0, S))
                window = set(range(i - R + 1, i + 1))
                if j not in sinks and j not in window:
                    continue
            keys.append(b)
        scores = [scale * sum(q[a][d] * k[b][d] for d in range(D)) for b in keys]
        top = max(scores)
        w = [math.exp(s - top) for s in scores]
        tot = sum(w)
        out.append([sum(w[n] * v[b][d] for n, b in enumerate(keys)) / tot for d in range(D)])
    return np.array(out)


@pytest.mark.parametrize("kind", ["full", "streaming"])
@pytest.mark.parametrize("seed", [0, 1, 2, 3])
def test_masked_attention_vs_brute_force(kind, seed):
    g = rng(seed)
    T = int(g.integers(1, 14))
    D = int(g.integers(1, 6))
    S = int(g.integers(0, 4))
    R = int(g.integers(1, 5))
    offset = int(g.integers(0, 9))          # chunk starting mid-sequence
    q = normal(g, (T, D)).astype(np.float64)
    k = normal(g, (T + offset, D)).astype(np.float64)
    v = normal(g, (T + offset, D)).astype(np.float64)
    q_pos = np.arange(offset, offset + T)
    k_pos = np.arange(T + offset)
    scale = 0.37
    got = oracle.masked_attention(q, k, v, q_pos, k_pos, scale, kind, S, R)
    ref = _brute(q.tolist(), k.tolist(), v.tolist(), q_pos, k_pos, scale, kind, S, R)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


def test_brute_force_with_permuted_keys():
    """Keys given out of position order (as a ring holds them)."""
    g = rng(7)
    T, D, S, R = 12, 3, 2, 3
    q = normal(g, (T, D)).astype(np.float64)
    k = normal(g, (T, D)).astype(np.float64)
    v = normal(g, (T, D)).astype(np.float64)
    perm = g.permutation(T)
    pos = np.arange(T)
    got = oracle.masked_attention(q, k[perm], v[perm], pos, pos[perm], 1.0, "streaming", S, R)
    ref = _brute(q.tolist(), k[perm].tolist(), v[perm].tolist(), pos, pos[perm], 1.0,
                 "streaming", S, R)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kind", ["full", "streaming"])
def test_vs_torch_sdpa_float64(kind):
    import torch
    g = rng(11)
    T, Hq, Hkv, D, S, R = 96, 4, 2, 16, 5, 9
    q = normal(g, (T, Hq, D)).astype(np.float64)
    k = normal(g, (T, Hkv, D)).astype(np.float64)
    v = normal(g, (T, Hkv, D)).astype(np.float64)
    scale = 0.25
    mask = np.ones(Hkv, np.uint8) if kind == "full" else np.zeros(Hkv, np.uint8)
    got = oracle.layer_attention(q, k, v, mask, scale, S, R)
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    allow = j <= i
    if kind == "streaming":
        allow = allow & ((j < S) | (i - j < R))
    G = Hq // Hkv
    for h in range(Hq):
        qt = torch.from_numpy(q[:, h])[None, None]
        kt = torch.from_numpy(k[:, h // G])[None, None]
        vt = torch.from_numpy(v[:, h // G])[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=torch.from_numpy(allow), scale=scale)[0, 0].numpy()
        np.testing.assert_allclose(got[:, h], ref, rtol=1e-10, atol=1e-12)


def test_single_token_returns_its_value():
    g = rng(3)
    q, k, v = (normal(g, (1, 8)).astype(np.float64) for _ in range(3))
    for kind in ("full", "streaming"):
        o = oracle.masked_attention(q, k, v, [0], [0], 0.5, kind, 16, 64)
        np.testing.assert_array_equal(o, v)


def test_zero_query_gives_prefix_mean():
    g = rng(4)
    T, D = 40, 5
    k = normal(g, (T, D)).astype(np.float64)
    v = normal(g, (T, D)).astype(np.float64)
    q = np.zeros((T, D))
    pos = np.arange(T)
    o = oracle.masked_attention(q, k, v, pos, pos, 1.0, "full")
    ref = np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None]
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-13)
    # streaming with S=3, R=4: mean over the sinks and the window
    o = oracle.masked_attention(q, k, v, pos, pos, 1.0, "streaming", 3, 4)
    for i in range(T):
        keys = sorted(set(range(min(3, i + 1))) | set(range(max(0, i - 3), i + 1)))
        np.testing.assert_allclose(o[i], v[keys].mean(axis=0), rtol=1e-12, atol=1e-13)


def test_window_of_one_returns_own_value():
    g = rng(5)
    T, D = 30, 4
    q, k, v = (normal(g, (T, D)).astype(np.float64) for _ in range(3))
    pos = np.arange(T)
    o = oracle.masked_attention(q, k, v, pos, pos, 1.0, "streaming", 0, 1)
    np.testing.assert_array_equal(o, v)


def test_planted_key_dominates():
    g = rng(6)
    T, D, planted = 64, 8, 20
    k = normal(g, (T, D)).astype(np.float64) * 0.1
    v = normal(g, (T, D)).astype(np.float64)
    q = np.zeros((T, D))
    q[:, 0] = 1.0
    k[planted, 0] = 60.0            # logit about 60 above every other key
    pos = np.arange(T)
    o = oracle.masked_attention(q, k, v, pos, pos, 1.0, "full")
    np.testing.assert_allclose(o[planted:], np.broadcast_to(v[planted], (T - planted, D)),
                               atol=1e-20 + 1e-12)
    # the streaming mask drops the planted key once it leaves the window
    o = oracle.masked_attention(q, k, v, pos, pos, 1.0, "streaming", 2, 8)
    assert np.abs(o[planted + 4] - v[planted]).max() < 1e-12
    assert np.abs(o[planted + 8] - v[planted]).max() > 1e-3


def test_window_covering_sequence_equals_full():
    g = rng(8)
    T, H, D = 50, 3, 8
    q, k, v = (normal(g, (T, H, D)).astype(np.float64) for _ in range(3))
    full = oracle.full_attention(q, k, v, 0.3)
    for S, R in [(0, T), (16, 64), (T, 1), (20, 30)]:
        st = oracle.streaming_attention(q, k, v, 0.3, S, R)
        np.testing.assert_array_equal(st, full)


def test_mixed_alpha_one_and_zero():
    g = rng(9)
    T, Hq, Hkv, D = 120, 4, 2, 8
    q = normal(g, (T, Hq, D)).astype(np.float64)
    k, v = (normal(g, (T, Hkv, D)).astype(np.float64) for _ in range(2))
    full = oracle.full_attention(q, k, v, 0.5)
    st = oracle.streaming_attention(q, k, v, 0.5, 4, 8)
    np.testing.assert_array_equal(oracle.mixed_attention(q, k, v, [1.0, 1.0], 0.5, 4, 8), full)
    np.testing.assert_array_equal(oracle.mixed_attention(q, k, v, [0.0, 0.0], 0.5, 4, 8), st)
    mix = oracle.mixed_attention(q, k, v, [1.0, 0.0], 0.5, 4, 8)
    np.testing.assert_array_equal(mix[:, :2], full[:, :2])
    np.testing.assert_array_equal(mix[:, 2:], st[:, 2:])
    # affine in alpha
    half = oracle.mixed_attention(q, k, v, [0.5, 0.25], 0.5, 4, 8)
    np.testing.assert_allclose(half[:, :2], 0.5 * (full[:, :2] + st[:, :2]), atol=1e-14)
    np.testing.assert_allclose(half[:, 2:], 0.25 * full[:, 2:] + 0.75 * st[:, 2:], atol=1e-14)
    # the streaming and full parts genuinely differ at this length
    assert np.abs(full - st).max() > 1e-2


def test_layer_routing_by_mask():
    g = rng(10)
    T, H, D = 90, 6, 4
    q, k, v = (normal(g, (T, H, D)).astype(np.float64) for _ in range(3))
    mask = np.array([1, 0, 0, 1, 0, 1], np.uint8)
    out = oracle.layer_attention(q, k, v, mask, 1.0, 2, 5)
    full = oracle.full_attention(q, k, v, 1.0)
    st = oracle.streaming_attention(q, k, v, 1.0, 2, 5)
    for h in range(H):
        np.testing.assert_array_equal(out[:, h], (full if mask[h] else st)[:, h])


def test_gqa_equals_replicated_mha():
    g = rng(12)
    T, Hkv, G, D = 70, 2, 4, 8
    q = normal(g, (T, Hkv * G, D)).astype(np.float64)
    k, v = (normal(g, (T, Hkv, D)).astype(np.float64) for _ in range(2))
    mask = np.array([1, 0], np.uint8)
    gqa = oracle.layer_attention(q, k, v, mask, 0.7, 3, 6)
    k_rep = np.repeat(k, G, axis=1)
    v_rep = np.repeat(v, G, axis=1)
    mha = oracle.layer_attention(q, k_rep, v_rep, np.repeat(mask, G), 0.7, 3, 6)
    np.testing.assert_array_equal(gqa, mha)


def test_no_allowed_key_is_an_error():
    with pytest.raises(ValueError):
        oracle.masked_attention(np.zeros((1, 2)), np.zeros((1, 2)), np.zeros((1, 2)),
                                [0], [5], 1.0, "full")


def test_mixed_rows_subset_matches_all_rows():
    g = rng(13)
    T, H, D = 100, 2, 4
    q, k, v = (normal(g, (T, H, D)).astype(np.float64) for _ in range(3))
    full = oracle.mixed_attention(q, k, v, [0.3, 0.8], 0.5, 3, 7)
    rows = [0, 17, 99]
    part = oracle.mixed_attention(q, k, v, [0.3, 0.8], 0.5, 3, 7, rows=rows)
    np.testing.assert_array_equal(part[rows], full[rows])
    assert np.isnan(part[1]).all()
