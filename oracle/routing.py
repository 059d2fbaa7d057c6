"""Head-split routing (test infrastructure; see package doc).

Before deployment the Q/K/V projection output channels are reordered so that
retrieval heads and streaming heads form two contiguous blocks, which makes
splitting and concatenating along the head axis plain slicing (xllm-io review,
section 三 模型部署优化). Reading: the order is stable -- retrieval KV heads in
ascending original index, then streaming KV heads in ascending index -- and
query heads move with their KV head in whole groups of G.
"""
from __future__ import annotations

import numpy as np


def head_permutation(mask):
    """mask [Hkv] (nonzero = retrieval) -> (perm, n_retrieval), where perm[i]
    is the original KV head placed at position i."""
    mask = [int(m) != 0 for m in mask]
    retrieval = [h for h, m in enumerate(mask) if m]
    streaming = [h for h, m in enumerate(mask) if not m]
    return retrieval + streaming, len(retrieval)


def invert_permutation(perm):
    inv = [0] * len(perm)
    for i, p in enumerate(perm):
        inv[p] = i
    return inv


def apply_head_permutation(x, kv_perm, axis: int, group: int = 1):
    """Reorder axis ``axis`` of x (length len(kv_perm) * group) so that block
    i of ``group`` heads is the original block kv_perm[i]."""
    x = np.asarray(x)
    idx = [p * group + g for p in kv_perm for g in range(group)]
    return np.take(x, idx, axis=axis)
