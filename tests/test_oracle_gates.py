"""Pins of the oracle's gate-identification pieces against things other than
themselves.

* the gradient with respect to the gates: finite differences of the oracle's
  gate-blended forward (the output is affine in each gate, so a unit step is
  exact), pure-Python brute force on tiny inputs, the pages' invariant that a
  window covering the whole sequence makes streaming equal full (zero data
  term), the L1 term alone when dout = 0, and GQA summing its query heads;
* binarization: hand-worked gates, the extremes 0 and 1, ties at the
  threshold, and the split property on random gates;
* the weight reorder: projecting with reordered rows equals reordering the
  projected heads, and the inverse permutation restores the weights.
"""
import math

import numpy as np
import pytest

import oracle
from duo_synth import rng, normal


def _inputs(T, Hq, Hkv, D, seed):
    g = rng(seed)
    q = normal(g, (T, Hq, D)).astype(np.float64)
    k = normal(g, (T, Hkv, D)).astype(np.float64)
    v = normal(g, (T, Hkv, D)).astype(np.float64)
    dout = normal(g, (T, Hq, D)).astype(np.float64)
    alpha = g.uniform(0.0, 1.0, Hkv)
    return q, k, v, dout, alpha


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (6, 2)])
def test_grad_is_the_forward_difference(Hq, Hkv):
    T, D, S, R = 40, 8, 3, 7
    q, k, v, dout, alpha = _inputs(T, Hq, Hkv, D, 9100 + Hq)
    scale = D ** -0.5
    grad = oracle.mixed_alpha_grad(q, k, v, dout, alpha, scale, S, R)
    base = np.sum(dout * oracle.mixed_attention(q, k, v, alpha, scale, S, R))
    for kv in range(Hkv):
        a1 = alpha.copy()
        a1[kv] += 1.0  # o is affine in the gate: the unit step is the derivative
        up = np.sum(dout * oracle.mixed_attention(q, k, v, a1, scale, S, R))
        assert abs((up - base) - grad[kv]) <= 1e-9 * (1.0 + abs(grad[kv]))


def _brute_row(qi, ks, vs, allowed, scale):
    logits = [scale * sum(a * b for a, b in zip(qi, kj)) for kj, ok in zip(ks, allowed) if ok]
    vals = [vj for vj, ok in zip(vs, allowed) if ok]
    m = max(logits)
    w = [math.exp(x - m) for x in logits]
    tot = sum(w)
    return [sum(wj * vj[d] for wj, vj in zip(w, vals)) / tot for d in range(len(qi))]


def test_grad_brute_force_tiny():
    T, Hq, Hkv, D, S, R = 9, 2, 1, 3, 2, 3
    q, k, v, dout, alpha = _inputs(T, Hq, Hkv, D, 9200)
    scale, lam = 0.7, 0.05
    want = 0.0
    for h in range(Hq):
        for i in range(T):
            full = [j <= i for j in range(T)]
            lam_m = [j <= i and (j < S or i - j < R) for j in range(T)]
            of = _brute_row(q[i, h], k[:, 0], v[:, 0], full, scale)
            os_ = _brute_row(q[i, h], k[:, 0], v[:, 0], lam_m, scale)
            want += sum(dout[i, h, d] * (of[d] - os_[d]) for d in range(D))
    want += lam * (1.0 if alpha[0] > 0 else 0.0)
    got = oracle.mixed_alpha_grad(q, k, v, dout, alpha, scale, S, R, l1_weight=lam)
    assert abs(got[0] - want) <= 1e-12 * (1.0 + abs(want))


def test_grad_zero_when_window_covers_sequence():
    T, S, R = 30, 10, 20  # S + R >= T: the Lambda mask keeps every causal key
    q, k, v, dout, alpha = _inputs(T, 4, 2, 8, 9300)
    grad = oracle.mixed_alpha_grad(q, k, v, dout, alpha, 0.35, S, R)
    assert np.all(grad == 0.0)


def test_grad_l1_term_alone():
    q, k, v, _, _ = _inputs(20, 4, 4, 8, 9400)
    alpha = np.array([0.3, 0.0, -0.2, 1.0])
    grad = oracle.mixed_alpha_grad(q, k, v, np.zeros((20, 4, 8)), alpha, 0.35, 2, 5,
                                   l1_weight=0.05)
    assert np.array_equal(grad, [0.05, 0.0, -0.05, 0.05])


def test_grad_gqa_sums_query_heads():
    T, D, S, R = 33, 8, 2, 6
    q, k, v, dout, alpha = _inputs(T, 6, 2, D, 9500)
    G = 3
    gqa = oracle.mixed_alpha_grad(q, k, v, dout, alpha, 0.4, S, R)
    # the same layer as MHA with K/V repeated per query head and one gate each
    k6, v6 = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    mha = oracle.mixed_alpha_grad(q, k6, v6, dout, np.repeat(alpha, G), 0.4, S, R)
    np.testing.assert_allclose(gqa, mha.reshape(2, G).sum(axis=1), rtol=1e-12, atol=1e-12)


def test_binarize_hand_examples():
    assert oracle.binarize_gates([0.9, 0.1, 0.5, 0.3], 0.5).tolist() == [1, 0, 1, 0]
    assert oracle.binarize_gates([0.9, 0.1, 0.5, 0.3], 0.0).tolist() == [1, 1, 1, 1]
    assert oracle.binarize_gates([0.9, 0.1, 0.5, 0.3], 1.0).tolist() == [0, 0, 0, 0]
    assert oracle.binarize_gates([0.9, 0.1, 0.5, 0.3], 0.74).tolist() == [1, 0, 1, 0]
    assert oracle.binarize_gates([0.9, 0.1, 0.5, 0.3], 0.75).tolist() == [1, 0, 0, 0]
    # gates tied with the threshold stay retrieval heads
    assert oracle.binarize_gates([0.5, 0.5, 0.5, 0.1], 0.5).tolist() == [1, 1, 1, 0]


def test_binarize_split_property():
    g = rng(9600)
    for _ in range(200):
        n = int(g.integers(1, 200))
        a = g.permutation(n) / n + g.uniform(0.0, 0.001)  # distinct gates
        s = float(g.uniform(0.0, 1.0))
        m = oracle.binarize_gates(a, s)
        k = int(np.floor(s * n))
        assert int((m == 0).sum()) == k
        if 0 < k < n:
            assert a[m == 0].max() < a[m == 1].min()


def test_reorder_rows_matches_reordered_heads():
    g = rng(9700)
    Hkv, G, D, hidden = 4, 2, 8, 24
    mask = np.array([0, 1, 0, 1], np.uint8)
    kv_perm, _ = oracle.head_permutation(mask)
    q_perm = (np.asarray(kv_perm)[:, None] * G + np.arange(G)[None, :]).ravel()
    wq = normal(g, (Hkv * G * D, hidden))
    x = normal(g, (5, hidden))
    heads = (x @ wq.T).reshape(5, Hkv * G, D)
    wq_r = oracle.reorder_head_rows(wq, q_perm, D)
    heads_r = (x @ wq_r.T).reshape(5, Hkv * G, D)
    np.testing.assert_array_equal(heads_r, heads[:, q_perm])
    inv = oracle.invert_permutation(q_perm)
    np.testing.assert_array_equal(oracle.reorder_head_rows(wq_r, inv, D), wq)
