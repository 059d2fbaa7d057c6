"""Pins of the oracle's head routing (xllm-io review, section 三 模型部署优化:
retrieval and streaming heads are made contiguous blocks).

* a hand-worked permutation for the 8-head workload with retrieval heads {0, 5};
* the permutation is a bijection, stable within each block, and its inverse
  restores the original order bit for bit;
* routing a layer through the permutation and back leaves the output equal to
  the unpermuted computation.
"""
import numpy as np

import oracle
from duo_synth import rng, normal


def test_hand_worked_example():
    perm, nr = oracle.head_permutation([1, 0, 0, 0, 0, 1, 0, 0])
    assert perm == [0, 5, 1, 2, 3, 4, 6, 7]
    assert nr == 2


def test_bijective_stable_and_invertible():
    g = rng(41)
    for _ in range(50):
        H = int(g.integers(1, 40))
        mask = g.integers(0, 2, size=H)
        perm, nr = oracle.head_permutation(mask)
        assert sorted(perm) == list(range(H))
        assert nr == int(mask.sum())
        assert all(mask[p] for p in perm[:nr]) and not any(mask[p] for p in perm[nr:])
        assert perm[:nr] == sorted(perm[:nr]) and perm[nr:] == sorted(perm[nr:])
        inv = oracle.invert_permutation(perm)
        x = g.standard_normal((3, H * 2, 5))
        y = oracle.apply_head_permutation(x, perm, axis=1, group=2)
        back = oracle.apply_head_permutation(y, inv, axis=1, group=2)
        np.testing.assert_array_equal(back, x)


def test_layer_output_commutes_with_routing():
    g = rng(42)
    T, Hkv, G, D = 60, 4, 2, 8
    q = normal(g, (T, Hkv * G, D)).astype(np.float64)
    k, v = (normal(g, (T, Hkv, D)).astype(np.float64) for _ in range(2))
    mask = np.array([0, 1, 0, 1], np.uint8)
    ref = oracle.layer_attention(q, k, v, mask, 0.5, 2, 6)
    perm, nr = oracle.head_permutation(mask)
    qp = oracle.apply_head_permutation(q, perm, 1, G)
    kp = oracle.apply_head_permutation(k, perm, 1)
    vp = oracle.apply_head_permutation(v, perm, 1)
    mp = np.array([1] * nr + [0] * (Hkv - nr), np.uint8)
    outp = oracle.layer_attention(qp, kp, vp, mp, 0.5, 2, 6)
    back = oracle.apply_head_permutation(outp, oracle.invert_permutation(perm), 1, G)
    np.testing.assert_array_equal(back, ref)
