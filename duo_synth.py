"""Seeded synthetic inputs for the DuoAttention hot path.

This module only draws random numbers and rounds them to the storage type the
kernels consume. It holds none of the method's arithmetic (no masks, no
softmax, no ring or quantisation logic), so both the CPU oracle's tests and the
GPU path may use it without sharing any computation.

Workloads. The pages measure whole models (Llama-2-7B-32K-Instruct,
Llama-3-8B-Instruct-Gradient-1048k) on NIAH and LongBench; those models and
suites are not available, so per-layer tensors of the same shapes stand in for
them: N(0,1) activations for Q/K/V, retrieval heads chosen by seed, alpha drawn
from U(0,1). N(0,1) inputs give diffuse attention; the needle inputs below add
one sharply peaked key for routing checks.

Recipe (host path). ``numpy.random.Generator(PCG64(seed))`` with
``seed = 1000 + config index`` draws, in this order: Q of the prefill or mixed
sequence (token-major ``[T, Hq, D]``); K and V of the prefill or context in
chunks of 65536 tokens (K chunk, then V chunk, ``[n, Hkv, D]`` each); the
per-step q, k, v of the decode steps (``[steps, H, D]`` each); alpha; then the
retrieval-head choice ``sorted(permutation(H_kv)[:H_r])``. Values are float32
standard normals rounded to bf16 (round-to-nearest-even) or, for the fp16 KV of
the 1M-token int4 decode workload, to fp16. ``ContextStream`` yields the same
sequence chunk by chunk for contexts too large to hold at once.

Recipe (device path, bench-scale only). ``torch.Generator(device=...)`` seeded
with the same seed fills large context tensors directly in HBM; such data is
never handed to the oracle.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

SEED_BASE = 1000


@dataclass(frozen=True)
class Workload:
    """Shape of one per-layer workload (batch 1)."""

    key: str
    index: int
    description: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_retrieval_kv: int
    sink: int = 16
    recent: int = 64
    softmax_scale: float = 1.0
    q_prescale: float = 1.0          # factor folded into Q at generation time
    prefill_tokens: int = 0          # tokens fed through chunked prefill
    chunk: int = 0                   # chunk length of the prefill
    context: int = 0                 # tokens appended (no attention) before decode
    decode_steps: int = 0
    mixed_tokens: int = 0            # sequence length of the alpha-blend forward
    fixed_retrieval: Optional[Sequence[int]] = None
    kv_dtype: str = "bf16"           # retrieval cache: bf16 | int4
    ring_dtype: str = "bf16"         # streaming ring: bf16 | fp16


WORKLOADS = {
    "mha8_d64_seq1024": Workload(
        key="mha8_d64_seq1024", index=0,
        description="MHA 8 heads, D=64, prefill 1024 as one chunk + 16 decode steps; "
                    "retrieval heads {0,5}",
        n_q_heads=8, n_kv_heads=8, head_dim=64, n_retrieval_kv=2,
        softmax_scale=1.0 / 8.0, prefill_tokens=1024, chunk=1024, decode_steps=16,
        fixed_retrieval=(0, 5)),
    "llama2_7b_decode_32k": Workload(
        key="llama2_7b_decode_32k", index=1,
        description="Llama-2-7B decode layer: MHA 32x128, 32768-token context, "
                    "8 retrieval heads, 256 decode steps",
        n_q_heads=32, n_kv_heads=32, head_dim=128, n_retrieval_kv=8,
        softmax_scale=1.0, q_prescale=1.0 / math.sqrt(128.0),
        context=32768, decode_steps=256),
    "llama3_8b_prefill_64k": Workload(
        key="llama3_8b_prefill_64k", index=2,
        description="Llama-3-8B GQA chunked prefill: 32q/8kv x 128, 65536 tokens in "
                    "8192-token chunks, 4 retrieval KV heads",
        n_q_heads=32, n_kv_heads=8, head_dim=128, n_retrieval_kv=4,
        softmax_scale=1.0 / math.sqrt(128.0), prefill_tokens=65536, chunk=8192),
    "llama2_7b_mixed_16k": Workload(
        key="llama2_7b_mixed_16k", index=3,
        description="alpha-blend mixed forward: MHA 32x128, seq 16384, alpha~U(0,1)",
        n_q_heads=32, n_kv_heads=32, head_dim=128, n_retrieval_kv=0,
        softmax_scale=1.0 / math.sqrt(128.0), mixed_tokens=16384),
    "llama3_8b_int4_decode_1m": Workload(
        key="llama3_8b_int4_decode_1m", index=4,
        description="Llama-3-8B GQA decode: 32q/8kv x 128, 1048576-token context, "
                    "4 int4 retrieval KV heads, fp16 ring, 64 decode steps",
        n_q_heads=32, n_kv_heads=8, head_dim=128, n_retrieval_kv=4,
        softmax_scale=1.0 / math.sqrt(128.0), context=1048576, decode_steps=64,
        kv_dtype="int4", ring_dtype="fp16"),
}

WORKLOAD_ORDER = [
    "mha8_d64_seq1024", "llama2_7b_decode_32k", "llama3_8b_prefill_64k",
    "llama2_7b_mixed_16k", "llama3_8b_int4_decode_1m",
]


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal(gen: np.random.Generator, shape) -> np.ndarray:
    return gen.standard_normal(size=shape, dtype=np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bf16 (ties to even), returned as float32 values."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.bfloat16).to(torch.float32).numpy()


def round_fp16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest fp16 (ties to even), returned as float32 values."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


def to_storage(x: np.ndarray, dtype: str):
    """Round float32 values to ``dtype`` and return (torch CPU tensor in that
    dtype, float64 numpy copy of exactly the stored values)."""
    import torch
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "bf16":
        t = torch.from_numpy(x).to(torch.bfloat16)
    elif dtype == "fp16":
        t = torch.from_numpy(x.astype(np.float16))
    elif dtype == "fp32":
        t = torch.from_numpy(x.copy())
    else:
        raise ValueError(dtype)
    return t, t.to(torch.float64).numpy()


def choose_retrieval(gen: np.random.Generator, n_kv_heads: int, n_retrieval: int):
    return sorted(int(h) for h in gen.permutation(n_kv_heads)[:n_retrieval])


def retrieval_mask_from_heads(n_kv_heads: int, heads: Sequence[int]) -> np.ndarray:
    m = np.zeros(n_kv_heads, dtype=np.uint8)
    m[list(heads)] = 1
    return m


@dataclass
class LayerInputs:
    """Seeded per-layer inputs in the caller's original head order."""

    workload: Workload
    retrieval_mask: np.ndarray            # [H_kv] u8, 1 = retrieval head
    q: Optional[np.ndarray] = None        # prefill / mixed: [T, Hq, D] float32 (rounded)
    k: Optional[np.ndarray] = None        # prefill / context: [T, Hkv, D]
    v: Optional[np.ndarray] = None
    q_steps: Optional[np.ndarray] = None  # [steps, Hq, D]
    k_steps: Optional[np.ndarray] = None  # [steps, Hkv, D]
    v_steps: Optional[np.ndarray] = None
    alpha: Optional[np.ndarray] = None    # [Hkv] float32
    extra: dict = field(default_factory=dict)


KV_CHUNK = 65536


class ContextStream:
    """The draw sequence of ``make_inputs``, produced chunk by chunk.

    Iterate ``chunks()`` to get (k, v) context/prefill chunks of up to
    ``KV_CHUNK`` tokens, then call ``tail()`` for the decode steps, alpha and
    the retrieval mask (in that draw order). ``q`` (prefill/mixed Q) is drawn
    up front."""

    def __init__(self, w: Workload, *, tokens: Optional[int] = None,
                 steps: Optional[int] = None, n_q_heads: Optional[int] = None,
                 seed: Optional[int] = None):
        self.w = w
        self.gen = rng(SEED_BASE + w.index if seed is None else seed)
        self.hq = w.n_q_heads if n_q_heads is None else n_q_heads
        self.T = tokens if tokens is not None else (w.prefill_tokens or w.context or w.mixed_tokens)
        self.steps = steps if steps is not None else w.decode_steps
        self.kv_round = round_fp16 if w.ring_dtype == "fp16" else round_bf16
        self.q = None
        if self.T and (w.prefill_tokens or w.mixed_tokens):
            self.q = round_bf16(normal(self.gen, (self.T, self.hq, w.head_dim))
                                * np.float32(w.q_prescale))

    def chunks(self):
        hkv, D = self.w.n_kv_heads, self.w.head_dim
        for a in range(0, self.T, KV_CHUNK):
            n = min(KV_CHUNK, self.T - a)
            k = self.kv_round(normal(self.gen, (n, hkv, D)))
            v = self.kv_round(normal(self.gen, (n, hkv, D)))
            yield k, v

    def tail(self, out: "LayerInputs") -> "LayerInputs":
        w, gen = self.w, self.gen
        hkv, D = w.n_kv_heads, w.head_dim
        if self.steps:
            out.q_steps = round_bf16(normal(gen, (self.steps, self.hq, D)) * np.float32(w.q_prescale))
            out.k_steps = self.kv_round(normal(gen, (self.steps, hkv, D)))
            out.v_steps = self.kv_round(normal(gen, (self.steps, hkv, D)))
        if w.mixed_tokens:
            out.alpha = gen.uniform(0.0, 1.0, size=hkv).astype(np.float32)
        if w.fixed_retrieval is not None:
            heads = list(w.fixed_retrieval)
        else:
            heads = choose_retrieval(gen, hkv, w.n_retrieval_kv)
        out.retrieval_mask = retrieval_mask_from_heads(hkv, heads)
        return out


def make_inputs(w: Workload, *, tokens: Optional[int] = None,
                steps: Optional[int] = None, n_q_heads: Optional[int] = None,
                seed: Optional[int] = None) -> LayerInputs:
    """Draw a workload's inputs on the host.

    ``tokens``/``steps`` override the prefill/context length and the decode
    step count (smaller cases of the same structure); the draw order is the
    one stated in the module docstring.
    """
    cs = ContextStream(w, tokens=tokens, steps=steps, n_q_heads=n_q_heads, seed=seed)
    out = LayerInputs(workload=w, retrieval_mask=np.zeros(w.n_kv_heads, np.uint8), q=cs.q)
    if cs.T:
        ks, vs = zip(*cs.chunks())
        out.k = ks[0] if len(ks) == 1 else np.concatenate(ks)
        out.v = vs[0] if len(vs) == 1 else np.concatenate(vs)
    return cs.tail(out)


def random_case(seed: int, *, T: int, n_q_heads: int, n_kv_heads: int, head_dim: int,
                kv_round=round_bf16):
    """Small generic case: (q [T,Hq,D], k [T,Hkv,D], v [T,Hkv,D]) rounded values."""
    gen = rng(seed)
    q = round_bf16(normal(gen, (T, n_q_heads, head_dim)))
    k = kv_round(normal(gen, (T, n_kv_heads, head_dim)))
    v = kv_round(normal(gen, (T, n_kv_heads, head_dim)))
    return q, k, v


def device_normal(shape, seed: int, device, dtype):
    """Bench-scale data drawn on the device (never given to the oracle)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32).to(dtype)
