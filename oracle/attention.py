"""Masked softmax attention in float64 (test infrastructure; see package doc).

Definitions followed:
  * full attention = softmax(Q K^T restricted to the causal mask) V, and
    streaming attention = the same under the Lambda mask that keeps only the
    initial (sink) tokens and the most recent tokens -- xllm-io review,
    section 三 技术架构, 核心公式.
  * mixed attention = alpha * full + (1 - alpha) * streaming with one gate per
    KV head -- xllm-io review, section 三 核心公式 (混合注意力) and 检索头识别;
    paperlayer summary, section 2 (Optimization-based Identification).
  * deployment sizes: 16 sink tokens and 64 recent tokens -- xllm-io review,
    section 五 消融实验 (item 3); paperlayer summary, section 3.

Readings (the pages leave these open):
  * the mask is a selection: disallowed scores are removed from the softmax
    (set to -inf), not multiplied by zero;
  * the softmax scale is an explicit argument (the printed formula has none);
  * "recent R" counts the query's own position: key j is recent for query i
    when i - j < R; sinks are the first S positions of the whole sequence;
  * query head h reads KV head h // G (G = query heads per KV head).
Masks are taken on absolute token positions, so a chunk or a ring cache is
handled by passing the positions its rows hold.

Block-sparse Lambda (the approximation used while training the gates --
paperlayer summary, appendix A.1; its figure is missing from the pages):
reading taken here, with block size b, query block i // b and key block
j // b: key j is allowed when j <= i and (its block is one of the first
ceil(S / b) blocks, or the query's block minus the key's block is below
ceil(R / b)). b = 1 is the token-level Lambda mask.
"""
from __future__ import annotations

import numpy as np


def allowed_mask(q_pos, k_pos, kind: str, sink: int, recent: int, block: int = 0) -> np.ndarray:
    """Boolean [len(q_pos), len(k_pos)]: may query position i attend key j.

    full:      j <= i
    streaming: j <= i and (j < sink or i - j < recent)   (the Lambda mask)
    streaming with block b > 0 (block-sparse Lambda):
               j <= i and (j // b < ceil(sink / b) or i // b - j // b < ceil(recent / b))
    """
    i = np.asarray(q_pos, dtype=np.int64)[:, None]
    j = np.asarray(k_pos, dtype=np.int64)[None, :]
    causal = j <= i
    if kind == "full":
        return causal
    if kind == "streaming":
        if block <= 0:
            return causal & ((j < sink) | (i - j < recent))
        sink_blocks = -(-sink // block)
        local_blocks = -(-recent // block)
        return causal & ((j // block < sink_blocks) | (i // block - j // block < local_blocks))
    raise ValueError(kind)


def masked_attention(q, k, v, q_pos, k_pos, scale: float, kind: str,
                     sink: int = 16, recent: int = 64, block: int = 0) -> np.ndarray:
    """o_i = sum_j p_ij v_j / sum_j p_ij over allowed j, p_ij = exp(s_ij - max_j s_ij),
    s_ij = scale * q_i . k_j.  q [Tq, D], k/v [Tk, D]; returns float64 [Tq, D]."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    s = scale * (q @ k.T)
    keep = allowed_mask(q_pos, k_pos, kind, sink, recent, block)
    if not keep.any(axis=1).all():
        raise ValueError("a query row has no allowed key")
    s = np.where(keep, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    return (p @ v) / l


def _group(n_q_heads: int, n_kv_heads: int) -> int:
    if n_q_heads % n_kv_heads:
        raise ValueError("query heads must be a multiple of KV heads")
    return n_q_heads // n_kv_heads


def layer_attention(q, k, v, retrieval_mask, scale: float, sink: int = 16,
                    recent: int = 64, q_pos=None, k_pos=None, heads=None) -> np.ndarray:
    """Head-split attention of one layer, in the caller's head order.

    q [Tq, Hq, D], k/v [Tk, Hkv, D]; retrieval_mask [Hkv] (nonzero = retrieval
    head, full attention; zero = streaming head, Lambda attention). Positions
    default to 0..T-1. ``heads`` restricts the query heads computed (others
    are left as NaN). Returns float64 [Tq, Hq, D].
    """
    q = np.asarray(q, dtype=np.float64)
    Tq, Hq, D = q.shape
    Tk, Hkv, _ = np.asarray(k).shape
    G = _group(Hq, Hkv)
    q_pos = np.arange(Tq) if q_pos is None else np.asarray(q_pos)
    k_pos = np.arange(Tk) if k_pos is None else np.asarray(k_pos)
    out = np.full((Tq, Hq, D), np.nan)
    for h in (range(Hq) if heads is None else heads):
        kv = h // G
        kind = "full" if retrieval_mask[kv] else "streaming"
        out[:, h] = masked_attention(q[:, h], k[:, kv], v[:, kv], q_pos, k_pos,
                                     scale, kind, sink, recent)
    return out


def full_attention(q, k, v, scale: float, q_pos=None, k_pos=None) -> np.ndarray:
    """Every head full causal: q [Tq,Hq,D], k/v [Tk,Hkv,D]."""
    hkv = np.asarray(k).shape[1]
    return layer_attention(q, k, v, np.ones(hkv, np.uint8), scale, q_pos=q_pos, k_pos=k_pos)


def streaming_attention(q, k, v, scale: float, sink: int = 16, recent: int = 64,
                        q_pos=None, k_pos=None) -> np.ndarray:
    """Every head Lambda-masked: q [Tq,Hq,D], k/v [Tk,Hkv,D]."""
    hkv = np.asarray(k).shape[1]
    return layer_attention(q, k, v, np.zeros(hkv, np.uint8), scale, sink, recent,
                           q_pos=q_pos, k_pos=k_pos)


def mixed_attention(q, k, v, alpha, scale: float, sink: int = 16, recent: int = 64,
                    heads=None, rows=None, block: int = 0) -> np.ndarray:
    """Gate-blended forward used for head identification:
    o_h = alpha[h // G] * full_h + (1 - alpha[h // G]) * streaming_h.
    q [T,Hq,D], k/v [T,Hkv,D], alpha [Hkv]; returns float64 [T,Hq,D].
    ``heads`` / ``rows`` restrict the query heads / rows computed (others NaN);
    ``block`` > 0 takes the streaming part under the block-sparse Lambda mask."""
    q = np.asarray(q, dtype=np.float64)
    T, Hq, D = q.shape
    Hkv = np.asarray(k).shape[1]
    G = _group(Hq, Hkv)
    pos = np.arange(T)
    rows = pos if rows is None else np.asarray(rows)
    out = np.full((T, Hq, D), np.nan)
    for h in (range(Hq) if heads is None else heads):
        kv = h // G
        a = float(alpha[kv])
        full = masked_attention(q[rows, h], k[:, kv], v[:, kv], rows, pos, scale, "full")
        stream = masked_attention(q[rows, h], k[:, kv], v[:, kv], rows, pos, scale,
                                  "streaming", sink, recent, block)
        out[rows, h] = a * full + (1.0 - a) * stream
    return out
