"""Gate identification pieces in float64 (test infrastructure; see package doc).

Definitions followed:
  * the gate-blended output o = alpha * full + (1 - alpha) * streaming, one
    gate per KV head shared by its query heads -- xllm-io review, section 三
    核心公式 (混合注意力); paperlayer summary, section 2 (Optimization-based
    Identification: GQA KV heads can serve several attention heads);
  * the loss L = L_distill + lambda * L_reg with L_reg the sum of |alpha| over
    the gates and lambda = 0.05 -- xllm-io review, section 三 核心公式
    (蒸馏损失, 正则化损失, 总损失); the model parameters stay fixed, only the
    gates are trained -- same section, 检索头识别 (step 2);
  * after training the gates are binarized: alpha = 1[alpha >= tau] -- xllm-io
    review, section 三 检索头识别 (step 3) -- with tau the sparsity quantile of
    the gate values -- paperlayer summary, section 2 (Binarizing Attention
    Implementations);
  * retrieval heads are made contiguous by reordering the heads' weight
    channels -- xllm-io review, section 三 模型部署优化.

Readings (the pages leave these open):
  * the attention layer's part of the gradient: with dout = dL_distill/do
    given, o is affine in each gate, so dL/dalpha_kv = sum over the tokens,
    the query heads of KV head kv and the channels of dout * (full -
    streaming), plus lambda * sign(alpha_kv) from the L1 term, with sign(0)
    taken as 0 (the subgradient 0);
  * the sparsity quantile: of N gates, k = floor(sparsity * N) become
    streaming heads; tau is the (k+1)-th smallest gate (tau = +inf when k = N),
    and a head is retrieval when alpha >= tau (gates tied with tau stay
    retrieval heads);
  * the weight reorder moves whole head blocks of output rows (D rows per
    head; a KV head's G query heads move together).
"""
from __future__ import annotations

import numpy as np

from .attention import masked_attention


def mixed_alpha_grad(q, k, v, dout, alpha, scale: float, sink: int = 16, recent: int = 64,
                     l1_weight: float = 0.0, block: int = 0) -> np.ndarray:
    """dL/dalpha for the gate-blended forward over one sequence.
    q [T,Hq,D], k/v [T,Hkv,D], dout [T,Hq,D] (dL_distill/do), alpha [Hkv];
    ``block`` > 0 takes the streaming part under the block-sparse Lambda mask;
    returns float64 [Hkv]."""
    q = np.asarray(q, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    T, Hq, D = q.shape
    Hkv = np.asarray(k).shape[1]
    if Hq % Hkv:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    G = Hq // Hkv
    pos = np.arange(T)
    grad = np.zeros(Hkv)
    for h in range(Hq):
        kv = h // G
        full = masked_attention(q[:, h], k[:, kv], v[:, kv], pos, pos, scale, "full")
        stream = masked_attention(q[:, h], k[:, kv], v[:, kv], pos, pos, scale, "streaming",
                                  sink, recent, block)
        grad[kv] += float(np.sum(dout[:, h] * (full - stream)))
    grad += l1_weight * np.sign(np.asarray(alpha, dtype=np.float64))
    return grad


def binarize_gates(alpha, sparsity: float) -> np.ndarray:
    """Retrieval mask (uint8, 1 = retrieval) from trained gates: the
    floor(sparsity * N) smallest gates become streaming heads, the threshold
    being the next gate in ascending order; gates tied with it stay
    retrieval heads."""
    a = np.asarray(alpha, dtype=np.float64).ravel()
    if not 0.0 <= sparsity <= 1.0:
        raise ValueError("sparsity must lie in [0, 1]")
    n = a.size
    n_stream = int(np.floor(sparsity * n))
    if n_stream >= n:
        return np.zeros(n, np.uint8)
    tau = np.sort(a, kind="stable")[n_stream]
    return (a >= tau).astype(np.uint8)


def reorder_head_rows(w, perm, rows_per_head: int) -> np.ndarray:
    """Rows of a projection weight grouped in head blocks of rows_per_head
    rows, moved so that block i of the result is block perm[i] of w."""
    w = np.asarray(w)
    perm = np.asarray(perm)
    n = perm.size
    if w.shape[0] != n * rows_per_head:
        raise ValueError("weight rows must be n_heads * rows_per_head")
    blocks = w.reshape((n, rows_per_head) + w.shape[1:])
    return blocks[perm].reshape(w.shape)
