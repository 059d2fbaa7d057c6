"""Two-cache layer state, chunked prefill and decode (test infrastructure).

What is followed:
  * each layer keeps two KV caches -- a full one for retrieval heads and one
    holding only sink and recent tokens for streaming heads; the new token's
    Q/K/V are split along the head axis, each block attends separately, and
    the outputs are concatenated along heads -- xllm-io review, section 三
    推理流程 (解码阶段);
  * prefill runs in fixed-length chunks that fill both caches; streaming heads
    need linear time and constant memory -- xllm-io review, section 三
    (预填充阶段); paperlayer summary, section 2 (Chunked Pre-filling).

Readings: the streaming cache is a ring of S + R slots; position p is stored
in slot p when p < S, else in slot S + ((p - S) mod R), and writes happen in
position order, so a later position overwrites an earlier one in its slot.
A decode step is a chunk of one token (append, then attend: the new token is
among its own keys). Keys keep their absolute positions; masks are taken on
those positions.
"""
from __future__ import annotations

import numpy as np

from .attention import masked_attention
from .int4 import quantize_int4_g32, dequantize_int4_g32


class _Rows:
    """Rows of one head's retrieval cache in a float64 array that grows by
    doubling (storage only: the rows are kept exactly as appended)."""

    def __init__(self, width):
        self.buf = np.empty((16, width), np.float64)
        self.n = 0

    def extend(self, rows):
        rows = np.asarray(rows, np.float64).reshape(-1, self.buf.shape[1])
        need = self.n + rows.shape[0]
        if need > self.buf.shape[0]:
            grown = np.empty((max(need, 2 * self.buf.shape[0]), self.buf.shape[1]), np.float64)
            grown[:self.n] = self.buf[:self.n]
            self.buf = grown
        self.buf[self.n:need] = rows
        self.n = need

    def rows(self):
        return self.buf[:self.n]

    def __len__(self):
        return self.n


def ring_slot(p: int, sink: int, recent: int) -> int:
    return p if p < sink else sink + (p - sink) % recent


def ring_positions_after(n_tokens: int, sink: int, recent: int):
    """Simulate position-ordered writes of positions 0..n-1 into the ring and
    return slot -> position (-1 = never written)."""
    slots = [-1] * (sink + recent)
    for p in range(n_tokens):
        slots[ring_slot(p, sink, recent)] = p
    return slots


class OracleLayer:
    """One attention layer's caches in the caller's head order.

    retrieval_mask [Hkv]: nonzero = retrieval head. int4=True stores the
    retrieval cache with the 4-bit group encoding of ``oracle.int4`` and
    attends over the dequantised values.
    """

    def __init__(self, n_q_heads, n_kv_heads, head_dim, retrieval_mask, scale,
                 sink=16, recent=64, int4=False):
        self.Hq, self.Hkv, self.D = n_q_heads, n_kv_heads, head_dim
        self.G = n_q_heads // n_kv_heads
        self.mask = [int(m) != 0 for m in retrieval_mask]
        self.scale, self.S, self.R = scale, sink, recent
        self.int4 = int4
        self.n = 0
        # retrieval heads: the rows the attention reads, in position order
        self.full_k = {h: _Rows(head_dim) for h in range(n_kv_heads) if self.mask[h]}
        self.full_v = {h: _Rows(head_dim) for h in range(n_kv_heads) if self.mask[h]}
        # int4 encodings kept for byte-level comparison: per head lists of (codes, s, z)
        self.enc_k = {h: [] for h in self.full_k}
        self.enc_v = {h: [] for h in self.full_k}
        # streaming heads: ring slots holding (position, k row, v row)
        self.ring = {h: [None] * (sink + recent) for h in range(n_kv_heads) if not self.mask[h]}

    # -- caches --------------------------------------------------------------
    def _store_retrieval(self, h, k_rows, v_rows):
        if self.int4:
            ck, sk, zk = quantize_int4_g32(k_rows)
            cv, sv, zv = quantize_int4_g32(v_rows)
            self.enc_k[h].append((ck, sk, zk))
            self.enc_v[h].append((cv, sv, zv))
            k_rows = dequantize_int4_g32(ck, sk, zk)
            v_rows = dequantize_int4_g32(cv, sv, zv)
        self.full_k[h].extend(k_rows)
        self.full_v[h].extend(v_rows)

    def _store_ring(self, k, v):
        """Position-ordered writes of tokens n..n+T-1 into the streaming rings."""
        for h in self.ring:
            for t in range(k.shape[0]):
                p = self.n + t
                self.ring[h][ring_slot(p, self.S, self.R)] = (
                    p, np.asarray(k[t, h], np.float64), np.asarray(v[t, h], np.float64))

    def append(self, k, v):
        """Append tokens n..n+T-1 to both caches (no attention). k/v [T,Hkv,D]."""
        k = np.asarray(k)
        v = np.asarray(v)
        for h in self.full_k:
            self._store_retrieval(h, k[:, h], v[:, h])
        self._store_ring(k, v)
        self.n += k.shape[0]

    def ring_contents(self, h):
        """slot -> position for streaming head h (-1 = empty)."""
        return [-1 if e is None else e[0] for e in self.ring[h]]

    # -- attention -------------------------------------------------------------
    def prefill_chunk(self, q, k, v, rows=None):
        """Chunk at positions n..n+T-1: q [T,Hq,D], k/v [T,Hkv,D] -> out [T,Hq,D].

        Retrieval heads attend causally over the full cache plus the chunk;
        streaming heads attend under the Lambda mask over the ring as it was
        before the chunk plus the chunk itself. Both caches are then updated.
        ``rows`` restricts the query rows computed (others NaN)."""
        q = np.asarray(q, np.float64)
        k = np.asarray(k, np.float64)
        v = np.asarray(v, np.float64)
        T = q.shape[0]
        chunk_pos = np.arange(self.n, self.n + T)
        rows = np.arange(T) if rows is None else np.asarray(rows)
        out = np.full((T, self.Hq, self.D), np.nan)
        for kvh in range(self.Hkv):
            if self.mask[kvh]:
                # the chunk joins the full cache first (4-bit caches hold its
                # decoded values), then its queries attend over positions
                # 0..n+T-1
                self._store_retrieval(kvh, k[:, kvh], v[:, kvh])
                keys = self.full_k[kvh].rows()
                vals = self.full_v[kvh].rows()
                k_pos = np.arange(self.n + T)
                kind = "full"
            else:
                held = [e for e in self.ring[kvh] if e is not None]
                keys = np.array([e[1] for e in held] + list(k[:, kvh])).reshape(-1, self.D)
                vals = np.array([e[2] for e in held] + list(v[:, kvh])).reshape(-1, self.D)
                k_pos = np.array([e[0] for e in held] + list(chunk_pos))
                kind = "streaming"
            for g in range(self.G):
                h = kvh * self.G + g
                out[rows, h] = masked_attention(q[rows, h], keys, vals, chunk_pos[rows], k_pos,
                                                self.scale, kind, self.S, self.R)
        # the rings are updated after every streaming head has read them
        self._store_ring(k, v)
        self.n += T
        return out

    def decode(self, q, k, v):
        """One new token: q [Hq,D], k/v [Hkv,D] -> out [Hq,D]."""
        return self.prefill_chunk(np.asarray(q)[None], np.asarray(k)[None],
                                  np.asarray(v)[None])[0]
