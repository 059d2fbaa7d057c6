"""Python binding of the C ABI: torch tensors provide device memory and
streams, the library does all the work.

``DuoLayer`` owns (as torch uint8 tensors) the retrieval cache, the streaming
ring and the workspace of one attention layer and forwards append / prefill /
decode calls to libduo.so. ``mixed_forward`` is the stateless gate-blended
forward. ``head_permutation`` and ``ring_slot`` are the host helpers.
"""
from __future__ import annotations

import ctypes
from ctypes import POINTER, byref, c_float, c_int32, c_int64, c_uint8, c_void_p
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import lib, check, make_desc, layout


def _stream_ptr(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _gpu(device) -> torch.device:
    """The device with its index resolved (the library has no host path)."""
    dev = torch.device(device)
    if dev.type != "cuda":
        raise ValueError(f"device {dev} is not a GPU")
    return dev if dev.index is not None else torch.device("cuda", torch.cuda.current_device())


def _check_act(t: torch.Tensor, name: str, shape, dtype, device: torch.device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_TORCH = {"bf16": torch.bfloat16, "fp16": torch.float16}


class DuoLayer:
    """One attention layer with a full cache for retrieval KV heads [0, Hr)
    and a sink + recent ring for streaming KV heads [Hr, Hkv)."""

    def __init__(self, *, n_q_heads: int, n_kv_heads: int, head_dim: int,
                 n_retrieval_kv_heads: int, capacity: int, softmax_scale: float,
                 sink: int = 16, recent: int = 64, batch: int = 1, kv_dtype: str = "bf16",
                 retrieval_dtype: Optional[str] = None, device="cuda",
                 n_tokens_existing=0):
        """n_tokens_existing: one count for every sequence, or a list of
        per-sequence counts (a ragged batch)."""
        self.desc = make_desc(batch=batch, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads,
                              head_dim=head_dim, n_retrieval_kv_heads=n_retrieval_kv_heads,
                              sink=sink, recent=recent, capacity=capacity, kv_dtype=kv_dtype,
                              retrieval_dtype=retrieval_dtype, softmax_scale=softmax_scale)
        self.layout = layout(self.desc)
        self.device = _gpu(device)
        self.B, self.Hq, self.Hkv, self.D = batch, n_q_heads, n_kv_heads, head_dim
        self.Hr, self.Hs = n_retrieval_kv_heads, n_kv_heads - n_retrieval_kv_heads
        self.G = n_q_heads // n_kv_heads
        self.S, self.R, self.capacity = sink, recent, capacity
        self.kv_dtype = kv_dtype
        self.retrieval_dtype = kv_dtype if retrieval_dtype is None else retrieval_dtype
        lay = self.layout
        self.rbuf = torch.zeros(max(lay.retrieval_bytes, 256), dtype=torch.uint8, device=self.device)
        self.sbuf = torch.zeros(max(lay.streaming_bytes, 256), dtype=torch.uint8, device=self.device)
        self.ws = torch.zeros(max(lay.workspace_bytes, 256), dtype=torch.uint8, device=self.device)
        h = c_void_p()
        if isinstance(n_tokens_existing, (list, tuple)):
            if len(n_tokens_existing) != batch:
                raise ValueError("n_tokens_existing needs one count per sequence")
            counts = (c_int64 * batch)(*[int(x) for x in n_tokens_existing])
            with torch.cuda.device(self.device):
                check(lib.duo_layer_init_ragged(byref(h), byref(self.desc), _ptr(self.rbuf),
                                                _ptr(self.sbuf), _ptr(self.ws), counts,
                                                _stream_ptr(self.device)), "duo_layer_init_ragged")
        else:
            with torch.cuda.device(self.device):
                check(lib.duo_layer_init(byref(h), byref(self.desc), _ptr(self.rbuf), _ptr(self.sbuf),
                                         _ptr(self.ws), int(n_tokens_existing),
                                         _stream_ptr(self.device)), "duo_layer_init")
        self._h = h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib.duo_layer_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def n_tokens(self) -> int:
        """Tokens cached: the largest count over the batch's sequences."""
        return int(lib.duo_layer_tokens(self._h))

    def sequence_tokens(self, b: int) -> int:
        return int(lib.duo_layer_sequence_tokens(self._h, int(b)))

    # -- calls -----------------------------------------------------------------
    def append_kv(self, k: torch.Tensor, v: torch.Tensor):
        T = k.shape[1]
        kvt = _TORCH[self.kv_dtype]
        _check_act(k, "k", (self.B, T, self.Hkv, self.D), kvt, self.device)
        _check_act(v, "v", (self.B, T, self.Hkv, self.D), kvt, self.device)
        with torch.cuda.device(self.device):
            check(lib.duo_append_kv(self._h, _ptr(k), _ptr(v), T, _stream_ptr(self.device)),
                  "duo_append_kv")

    def prefill_chunk(self, q, k, v, out=None):
        T = q.shape[1]
        kvt = _TORCH[self.kv_dtype]
        _check_act(q, "q", (self.B, T, self.Hq, self.D), torch.bfloat16, self.device)
        _check_act(k, "k", (self.B, T, self.Hkv, self.D), kvt, self.device)
        _check_act(v, "v", (self.B, T, self.Hkv, self.D), kvt, self.device)
        if out is None:
            out = torch.empty_like(q)
        _check_act(out, "out", (self.B, T, self.Hq, self.D), torch.bfloat16, self.device)
        with torch.cuda.device(self.device):
            check(lib.duo_prefill_chunk(self._h, _ptr(q), _ptr(k), _ptr(v), T, _ptr(out),
                                        _stream_ptr(self.device)), "duo_prefill_chunk")
        return out

    def append_kv_seq(self, b: int, k: torch.Tensor, v: torch.Tensor):
        """Append to sequence b alone: k/v [1, T, Hkv, D]."""
        T = k.shape[1]
        kvt = _TORCH[self.kv_dtype]
        _check_act(k, "k", (1, T, self.Hkv, self.D), kvt, self.device)
        _check_act(v, "v", (1, T, self.Hkv, self.D), kvt, self.device)
        with torch.cuda.device(self.device):
            check(lib.duo_append_kv_seq(self._h, int(b), _ptr(k), _ptr(v), T,
                                        _stream_ptr(self.device)), "duo_append_kv_seq")

    def prefill_chunk_seq(self, b: int, q, k, v, out=None):
        """Prefill a chunk of sequence b alone: q [1, T, Hq, D], k/v [1, T, Hkv, D]."""
        T = q.shape[1]
        kvt = _TORCH[self.kv_dtype]
        _check_act(q, "q", (1, T, self.Hq, self.D), torch.bfloat16, self.device)
        _check_act(k, "k", (1, T, self.Hkv, self.D), kvt, self.device)
        _check_act(v, "v", (1, T, self.Hkv, self.D), kvt, self.device)
        if out is None:
            out = torch.empty_like(q)
        _check_act(out, "out", (1, T, self.Hq, self.D), torch.bfloat16, self.device)
        with torch.cuda.device(self.device):
            check(lib.duo_prefill_chunk_seq(self._h, int(b), _ptr(q), _ptr(k), _ptr(v), T, _ptr(out),
                                            _stream_ptr(self.device)), "duo_prefill_chunk_seq")
        return out

    def decode(self, q, k, v, out=None):
        kvt = _TORCH[self.kv_dtype]
        _check_act(q, "q", (self.B, 1, self.Hq, self.D), torch.bfloat16, self.device)
        _check_act(k, "k", (self.B, 1, self.Hkv, self.D), kvt, self.device)
        _check_act(v, "v", (self.B, 1, self.Hkv, self.D), kvt, self.device)
        if out is None:
            out = torch.empty_like(q)
        _check_act(out, "out", (self.B, 1, self.Hq, self.D), torch.bfloat16, self.device)
        with torch.cuda.device(self.device):
            check(lib.duo_decode(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                 _stream_ptr(self.device)), "duo_decode")
        return out

    # -- views of the caller-owned caches (documented layout) -------------------
    def retrieval_kv(self):
        """(K, V) views [B, Hr, cap, D] of a bf16/fp16 retrieval cache."""
        assert self.retrieval_dtype != "int4"
        dt = _TORCH[self.kv_dtype]
        shape = (self.B, self.Hr, self.capacity, self.D)
        return (_bytes_view(self.rbuf, self.layout.k_offset, shape, dt),
                _bytes_view(self.rbuf, self.layout.v_offset, shape, dt))

    def retrieval_int4(self):
        """Views of a 4-bit retrieval cache (cap32 = capacity rounded up to 32):
        K codes [B,Hr,cap32,D/2] u8 (token-major, byte b = channel 2b | 2b+1 << 4),
        V codes [B,Hr,cap32/32,16*D] u8 (32-token blocks; channel ch, tokens m
        (low nibble) and m+16 (high nibble) of a block sit at byte
        16*(4*(16*(ch//64) + ch%16) + m//4) + 4*((ch%64)//16) + m%4), K and V
        scale/zero [B,Hr,cap32/32,D/32,32,2] fp16 (block, group, token in block)."""
        assert self.retrieval_dtype == "int4"
        cap32 = (self.capacity + 31) // 32 * 32
        ks = (self.B, self.Hr, cap32, self.D // 2)
        vs = (self.B, self.Hr, cap32 // 32, 16 * self.D)
        ss = (self.B, self.Hr, cap32 // 32, self.D // 32, 32, 2)
        return (_bytes_view(self.rbuf, self.layout.k_offset, ks, torch.uint8),
                _bytes_view(self.rbuf, self.layout.v_offset, vs, torch.uint8),
                _bytes_view(self.rbuf, self.layout.k_sz_offset, ss, torch.float16),
                _bytes_view(self.rbuf, self.layout.v_sz_offset, ss, torch.float16))

    def ring_kv(self):
        """(K, V) views [B, Hs, S+R, D] of the streaming ring."""
        dt = _TORCH[self.kv_dtype]
        shape = (self.B, self.Hs, self.S + self.R, self.D)
        return (_bytes_view(self.sbuf, self.layout.ring_k_offset, shape, dt),
                _bytes_view(self.sbuf, self.layout.ring_v_offset, shape, dt))


def _bytes_view(buf: torch.Tensor, offset: int, shape, dtype) -> torch.Tensor:
    n = 1
    for s in shape:
        n *= s
    nbytes = n * torch.empty((), dtype=dtype).element_size()
    return buf[offset:offset + nbytes].view(dtype).view(*shape)


def mixed_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, alpha: torch.Tensor, *,
                  softmax_scale: float, sink: int = 16, recent: int = 64, out=None,
                  lambda_block: int = 0):
    """out_h = alpha[h // G] * full_h + (1 - alpha[h // G]) * streaming_h.
    q [B,T,Hq,D] bf16, k/v [B,T,Hkv,D] bf16, alpha [Hkv] fp32 (device).
    lambda_block = 64 takes the streaming part under the block-sparse mask."""
    dev = _gpu(q.device)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    _check_act(q, "q", (B, T, Hq, D), torch.bfloat16, dev)
    _check_act(k, "k", (B, T, Hkv, D), torch.bfloat16, dev)
    _check_act(v, "v", (B, T, Hkv, D), torch.bfloat16, dev)
    _check_act(alpha, "alpha", (Hkv,), torch.float32, dev)
    if out is None:
        out = torch.empty_like(q)
    _check_act(out, "out", (B, T, Hq, D), torch.bfloat16, dev)
    desc = make_desc(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, n_retrieval_kv_heads=0,
                     sink=sink, recent=recent, capacity=0, softmax_scale=softmax_scale)
    with torch.cuda.device(dev):
        check(lib.duo_mixed_forward_block(byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), T,
                                          int(lambda_block), _ptr(out), _stream_ptr(dev)),
              "duo_mixed_forward_block")
    return out


def mixed_alpha_grad(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, dout: torch.Tensor,
                     alpha: torch.Tensor, *, softmax_scale: float, sink: int = 16,
                     recent: int = 64, l1_weight: float = 0.0, grad=None, workspace=None,
                     lambda_block: int = 0):
    """Gradient with respect to the gates of mixed_forward:
    grad[kv] = sum of dout * (full - streaming) over the batch, tokens, the
    query heads of KV head kv and channels, + l1_weight * sign(alpha[kv]).
    dout [B,T,Hq,D] bf16; returns grad [Hkv] fp32 (device). The workspace
    (uint8 device tensor) is allocated here unless given."""
    dev = _gpu(q.device)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    _check_act(q, "q", (B, T, Hq, D), torch.bfloat16, dev)
    _check_act(k, "k", (B, T, Hkv, D), torch.bfloat16, dev)
    _check_act(v, "v", (B, T, Hkv, D), torch.bfloat16, dev)
    _check_act(dout, "dout", (B, T, Hq, D), torch.bfloat16, dev)
    _check_act(alpha, "alpha", (Hkv,), torch.float32, dev)
    if grad is None:
        grad = torch.empty(Hkv, dtype=torch.float32, device=q.device)
    _check_act(grad, "grad", (Hkv,), torch.float32, dev)
    desc = make_desc(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, n_retrieval_kv_heads=0,
                     sink=sink, recent=recent, capacity=0, softmax_scale=softmax_scale)
    need = int(lib.duo_mixed_alpha_grad_workspace(byref(desc), T))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    _check_act(workspace, "workspace", (workspace.numel(),), torch.uint8, dev)
    with torch.cuda.device(dev):
        check(lib.duo_mixed_alpha_grad_block(byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                             _ptr(alpha), float(l1_weight), T, int(lambda_block),
                                             _ptr(grad), _ptr(workspace), workspace.numel(),
                                             _stream_ptr(dev)),
              "duo_mixed_alpha_grad_block")
    return grad


def mixed_alpha_grad_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                             dout: torch.Tensor, alpha: torch.Tensor, grad: torch.Tensor, *,
                             softmax_scale: float, sink: int = 16, recent: int = 64,
                             l1_weight: float = 0.0, lambda_block: int = 0):
    """mixed_alpha_grad through the entry point that allocates nothing: the
    per-block partial sums live in the library's device array (calls that
    overlap on one device race). The caller passes the output ``grad``
    [Hkv] fp32; a launch needing more than DUO_GRAD_SCRATCH_PARTIALS partial
    slots raises DuoError (status DUO_ERR_CAPACITY)."""
    dev = _gpu(q.device)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    _check_act(q, "q", (B, T, Hq, D), torch.bfloat16, dev)
    _check_act(k, "k", (B, T, Hkv, D), torch.bfloat16, dev)
    _check_act(v, "v", (B, T, Hkv, D), torch.bfloat16, dev)
    _check_act(dout, "dout", (B, T, Hq, D), torch.bfloat16, dev)
    _check_act(alpha, "alpha", (Hkv,), torch.float32, dev)
    _check_act(grad, "grad", (Hkv,), torch.float32, dev)
    desc = make_desc(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, n_retrieval_kv_heads=0,
                     sink=sink, recent=recent, capacity=0, softmax_scale=softmax_scale)
    with torch.cuda.device(dev):
        check(lib.duo_mixed_alpha_grad_noalloc(byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(dout),
                                               _ptr(alpha), float(l1_weight), T,
                                               int(lambda_block), _ptr(grad), _stream_ptr(dev)),
              "duo_mixed_alpha_grad_noalloc")
    return grad


def binarize_gates(alpha, sparsity: float):
    """Retrieval mask (list of 0/1, 1 = retrieval) from trained gates (host
    call): the floor(sparsity * n) smallest gates become streaming heads,
    gates tied with the threshold stay retrieval heads."""
    import numpy as np
    if isinstance(alpha, torch.Tensor):
        alpha = alpha.detach().to("cpu", torch.float32).numpy()
    a = np.ascontiguousarray(np.asarray(alpha, dtype=np.float32).ravel())
    n = int(a.size)
    mask = (c_uint8 * max(n, 1))()
    check(lib.duo_binarize_gates(a.ctypes.data_as(POINTER(c_float)), n, float(sparsity), mask),
          "duo_binarize_gates")
    return list(mask)[:n]


def reorder_head_rows(w, perm: Sequence[int], rows_per_head: int):
    """Host copy of a weight whose rows form head blocks of rows_per_head rows,
    with block i of the result = block perm[i] of w (numpy array or CPU
    tensor in, numpy array out)."""
    import numpy as np
    if isinstance(w, torch.Tensor):
        w = w.detach().cpu().numpy()
    src = np.ascontiguousarray(w)
    n = len(perm)
    if src.ndim < 1 or n < 1 or src.shape[0] != n * rows_per_head:
        raise ValueError("weight rows must be n_heads * rows_per_head")
    dst = np.empty_like(src)
    row_bytes = src.nbytes // src.shape[0]
    p = (c_int32 * n)(*[int(x) for x in perm])
    check(lib.duo_reorder_head_rows(src.ctypes.data, dst.ctypes.data, p, n, int(rows_per_head),
                                    int(row_bytes)), "duo_reorder_head_rows")
    return dst


def head_permutation(mask: Sequence[int]):
    """Stable permutation making retrieval KV heads contiguous (host call).
    Returns (perm, n_retrieval): perm[i] = original KV head at position i."""
    n = len(mask)
    m = (c_uint8 * n)(*[1 if x else 0 for x in mask])
    perm = (c_int32 * n)()
    nr = c_int32()
    check(lib.duo_head_permutation(m, n, perm, byref(nr)), "duo_head_permutation")
    return list(perm), int(nr.value)


def ring_slot(position: int, sink: int, recent: int) -> int:
    return int(lib.duo_ring_slot(position, sink, recent))
