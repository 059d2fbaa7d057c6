"""Pins of the oracle's block-sparse Lambda mask (the training-time
approximation of streaming attention; reading stated in oracle/attention.py)
against things other than itself:

* block size 1 is the token-level Lambda mask;
* hand-derived key sets for small cases;
* a covering case (every block local) equals full causal attention;
* pure-Python attention over key sets built as ranges of allowed blocks;
* the gate-blended forward's invariants under the block mask (alpha = 1 is
  full, alpha = 0 the block-streaming attention) and the gate gradient as the
  forward difference.
"""
import math

import numpy as np
import pytest

import oracle
from duo_synth import rng, normal


def _keys(mask_row):
    return [int(j) for j in np.nonzero(mask_row)[0]]


def test_block_one_is_token_lambda():
    g = rng(9800)
    for _ in range(100):
        T = int(g.integers(1, 90))
        S, R = int(g.integers(0, 20)), int(g.integers(1, 40))
        pos = np.arange(T)
        a = oracle.allowed_mask(pos, pos, "streaming", S, R)
        b = oracle.allowed_mask(pos, pos, "streaming", S, R, block=1)
        assert np.array_equal(a, b)


def test_hand_derived_key_sets():
    pos = np.arange(12)
    m = oracle.allowed_mask(pos, pos, "streaming", 2, 3, block=4)  # 1 sink block, 1 local block
    assert _keys(m[11]) == [0, 1, 2, 3, 8, 9, 10, 11]
    assert _keys(m[5]) == [0, 1, 2, 3, 4, 5]
    assert _keys(m[2]) == [0, 1, 2]
    assert _keys(m[8]) == [0, 1, 2, 3, 8]
    m = oracle.allowed_mask(pos, pos, "streaming", 5, 5, block=4)  # 2 sink blocks, 2 local blocks
    assert _keys(m[11]) == list(range(12))
    m = oracle.allowed_mask(np.arange(20), np.arange(20), "streaming", 0, 4, block=4)
    assert _keys(m[19]) == [16, 17, 18, 19]
    assert _keys(m[16]) == [16]


def test_covering_blocks_equal_full():
    pos = np.arange(50)
    # ceil(70 / 16) = 5 local blocks cover blocks 0..3 of a 50-token sequence
    m = oracle.allowed_mask(pos, pos, "streaming", 0, 70, block=16)
    assert np.array_equal(m, oracle.allowed_mask(pos, pos, "full", 0, 70))


def _brute_block(q, k, v, scale, S, R, b):
    T, D = q.shape
    sb, rb = -(-S // b), -(-R // b)
    out = np.zeros((T, D))
    for i in range(T):
        qb = i // b
        keys = set(range(0, min(sb * b, i + 1)))
        keys |= set(range(max(0, (qb - rb + 1) * b), i + 1))
        keys = sorted(keys)
        logits = [scale * sum(q[i, d] * k[j, d] for d in range(D)) for j in keys]
        m = max(logits)
        w = [math.exp(x - m) for x in logits]
        tot = sum(w)
        for d in range(D):
            out[i, d] = sum(wj * v[j, d] for wj, j in zip(w, keys)) / tot
    return out


@pytest.mark.parametrize("S,R,b", [(2, 3, 4), (0, 5, 4), (7, 1, 3), (16, 64, 8)])
def test_block_attention_brute_force(S, R, b):
    g = rng(9900 + S + R + b)
    T, D = 37, 4
    q, k, v = (normal(g, (T, D)).astype(np.float64) for _ in range(3))
    got = oracle.masked_attention(q, k, v, np.arange(T), np.arange(T), 0.6, "streaming", S, R,
                                  block=b)
    np.testing.assert_allclose(got, _brute_block(q, k, v, 0.6, S, R, b), rtol=1e-12, atol=1e-12)


def test_mixed_and_grad_under_block_mask():
    g = rng(9950)
    T, Hq, Hkv, D, S, R, b = 70, 4, 2, 8, 5, 9, 16
    q = normal(g, (T, Hq, D)).astype(np.float64)
    k = normal(g, (T, Hkv, D)).astype(np.float64)
    v = normal(g, (T, Hkv, D)).astype(np.float64)
    dout = normal(g, (T, Hq, D)).astype(np.float64)
    alpha = np.array([0.3, 0.8])
    one = oracle.mixed_attention(q, k, v, np.ones(Hkv), 0.3, S, R, block=b)
    zero = oracle.mixed_attention(q, k, v, np.zeros(Hkv), 0.3, S, R, block=b)
    np.testing.assert_allclose(one, oracle.full_attention(q, k, v, 0.3), rtol=1e-13, atol=1e-13)
    for h in range(Hq):
        ref = oracle.masked_attention(q[:, h], k[:, h // 2], v[:, h // 2], np.arange(T),
                                      np.arange(T), 0.3, "streaming", S, R, block=b)
        np.testing.assert_allclose(zero[:, h], ref, rtol=1e-13, atol=1e-13)
    grad = oracle.mixed_alpha_grad(q, k, v, dout, alpha, 0.3, S, R, block=b)
    base = np.sum(dout * oracle.mixed_attention(q, k, v, alpha, 0.3, S, R, block=b))
    for kv in range(Hkv):
        a1 = alpha.copy()
        a1[kv] += 1.0
        up = np.sum(dout * oracle.mixed_attention(q, k, v, a1, 0.3, S, R, block=b))
        assert abs((up - base) - grad[kv]) <= 1e-9 * (1.0 + abs(grad[kv]))
