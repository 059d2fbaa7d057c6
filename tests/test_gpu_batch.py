"""GPU parity with several sequences per launch, each with its own data (the
other batch tests repeat one sequence): context append + decode on the bf16
cache and on the 4-bit cache, chunked prefill followed by decode, and the
gate-blended mixed forward. Every batch element is compared with an oracle
that sees only that element's inputs."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from duo_synth import WORKLOADS, make_inputs, round_fp16
from gpu_util import Routed, assert_blocks_close, assert_close, device, say, to_dev

pytestmark = pytest.mark.gpu


def _batch_inputs(w, B, *, tokens, steps, seed):
    return [make_inputs(w, tokens=tokens, steps=steps, seed=seed + 101 * b) for b in range(B)]


def _stack(arrs, route, dtype):
    return torch.stack([route(to_dev(x, dtype)) for x in arrs]).contiguous()


def _layer(w, mask, B, capacity, kv_dtype="bf16", retrieval_dtype=None):
    import kv_cache_compression_duo_amd as duo
    G = w.n_q_heads // w.n_kv_heads
    r = Routed(mask, G)
    kw = {} if retrieval_dtype is None else {"retrieval_dtype": retrieval_dtype}
    lay = duo.DuoLayer(n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                       n_retrieval_kv_heads=r.nr, capacity=capacity,
                       softmax_scale=w.softmax_scale, sink=w.sink, recent=w.recent, batch=B,
                       kv_dtype=kv_dtype, device=device(), **kw)
    return lay, r


def _decode_steps(lay, r, inps, orcs, steps, dtype, rq, label):
    for s in range(steps):
        q = torch.stack([r.q(to_dev(x.q_steps[s]))[None] for x in inps]).contiguous()
        k = torch.stack([r.kv(to_dev(x.k_steps[s], dtype))[None] for x in inps]).contiguous()
        v = torch.stack([r.kv(to_dev(x.v_steps[s], dtype))[None] for x in inps]).contiguous()
        got = r.out(lay.decode(q, k, v)).float().cpu().numpy()
        for b, (x, o) in enumerate(zip(inps, orcs)):
            ref = o.decode(x.q_steps[s], x.k_steps[s], x.v_steps[s])
            assert_blocks_close(got[b, 0], ref, rq, f"{label} step {s} b{b}", head_axis=0)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp16"])
def test_decode_batch3_distinct(kv_dtype):
    w = dataclasses.replace(WORKLOADS["llama2_7b_decode_32k"], n_q_heads=8, n_kv_heads=8,
                            fixed_retrieval=(1, 4, 6))
    B, ctx, steps = 3, 900, 3
    say(f"case: decode batch {B}, {kv_dtype} cache, context {ctx}, distinct sequences")
    inps = _batch_inputs(w, B, tokens=ctx, steps=steps, seed=12000)
    mask = inps[0].retrieval_mask
    assert all((x.retrieval_mask == mask).all() for x in inps)
    dtype = torch.bfloat16 if kv_dtype == "bf16" else torch.float16
    if kv_dtype == "fp16":  # the oracle sees exactly the values the cache holds
        for x in inps:
            x.k, x.v = round_fp16(x.k), round_fp16(x.v)
            x.k_steps, x.v_steps = round_fp16(x.k_steps), round_fp16(x.v_steps)
    lay, r = _layer(w, mask, B, ctx + steps, kv_dtype=kv_dtype)
    lay.append_kv(_stack([x.k for x in inps], r.kv, dtype), _stack([x.v for x in inps], r.kv, dtype))
    orcs = []
    for x in inps:
        o = oracle.OracleLayer(w.n_q_heads, w.n_kv_heads, w.head_dim, mask, w.softmax_scale,
                               w.sink, w.recent)
        o.append(x.k, x.v)
        orcs.append(o)
    G = w.n_q_heads // w.n_kv_heads
    rq = np.array([mask[h // G] for h in range(w.n_q_heads)], bool)
    _decode_steps(lay, r, inps, orcs, steps, dtype, rq, f"decode-b{B}-{kv_dtype}")


def test_int4_decode_batch2_distinct():
    w = dataclasses.replace(WORKLOADS["llama3_8b_int4_decode_1m"], fixed_retrieval=(0, 3, 5, 6))
    B, ctx, steps = 2, 1000, 3
    say(f"case: 4-bit decode batch {B}, context {ctx}, distinct sequences")
    inps = _batch_inputs(w, B, tokens=ctx, steps=steps, seed=13000)
    mask = inps[0].retrieval_mask
    assert all((x.retrieval_mask == mask).all() for x in inps)
    dtype = torch.float16
    lay, r = _layer(w, mask, B, ctx + steps, kv_dtype="fp16", retrieval_dtype="int4")
    lay.append_kv(_stack([x.k for x in inps], r.kv, dtype), _stack([x.v for x in inps], r.kv, dtype))
    orcs = []
    for x in inps:
        o = oracle.OracleLayer(w.n_q_heads, w.n_kv_heads, w.head_dim, mask, w.softmax_scale,
                               w.sink, w.recent, int4=True)
        o.append(x.k, x.v)
        orcs.append(o)
    G = w.n_q_heads // w.n_kv_heads
    rq = np.array([mask[h // G] for h in range(w.n_q_heads)], bool)
    _decode_steps(lay, r, inps, orcs, steps, dtype, rq, f"int4-b{B}")


def test_prefill_batch2_distinct_then_decode():
    w = dataclasses.replace(WORKLOADS["llama3_8b_prefill_64k"], n_q_heads=16, n_kv_heads=4,
                            fixed_retrieval=(1, 2))
    B, chunks, steps = 2, [300, 211], 2
    T = sum(chunks)
    say(f"case: prefill batch {B}, chunks {chunks}, then {steps} decode steps, distinct sequences")
    inps = _batch_inputs(w, B, tokens=T, steps=steps, seed=14000)
    mask = inps[0].retrieval_mask
    assert all((x.retrieval_mask == mask).all() for x in inps)
    lay, r = _layer(w, mask, B, T + steps)
    orcs = [oracle.OracleLayer(w.n_q_heads, w.n_kv_heads, w.head_dim, mask, w.softmax_scale,
                               w.sink, w.recent) for _ in range(B)]
    G = w.n_q_heads // w.n_kv_heads
    rq = np.array([mask[h // G] for h in range(w.n_q_heads)], bool)
    a = 0
    for c in chunks:
        q = _stack([x.q[a:a + c] for x in inps], r.q, torch.bfloat16)
        k = _stack([x.k[a:a + c] for x in inps], r.kv, torch.bfloat16)
        v = _stack([x.v[a:a + c] for x in inps], r.kv, torch.bfloat16)
        got = r.out(lay.prefill_chunk(q, k, v)).float().cpu().numpy()
        for b, (x, o) in enumerate(zip(inps, orcs)):
            ref = o.prefill_chunk(x.q[a:a + c], x.k[a:a + c], x.v[a:a + c])
            assert_blocks_close(got[b], ref, rq, f"prefill-b{B} chunk@{a}+{c} b{b}", head_axis=1)
        a += c
    _decode_steps(lay, r, inps, orcs, steps, torch.bfloat16, rq, f"prefill-b{B} decode")


def test_mixed_batch2_distinct():
    import kv_cache_compression_duo_amd as duo
    w = dataclasses.replace(WORKLOADS["llama2_7b_mixed_16k"], n_q_heads=8, n_kv_heads=4)
    B, T = 2, 333
    say(f"case: mixed forward batch {B}, T={T}, distinct sequences")
    inps = _batch_inputs(w, B, tokens=T, steps=0, seed=15000)
    alpha = inps[0].alpha
    ident = lambda t: t  # noqa: E731 -- heads stay in the caller's order here
    q = _stack([x.q for x in inps], ident, torch.bfloat16)
    k = _stack([x.k for x in inps], ident, torch.bfloat16)
    v = _stack([x.v for x in inps], ident, torch.bfloat16)
    a = torch.from_numpy(np.asarray(alpha, np.float32)).to(device())
    got = duo.mixed_forward(q, k, v, a, softmax_scale=w.softmax_scale, sink=w.sink,
                            recent=w.recent).float().cpu().numpy()
    for b, x in enumerate(inps):
        ref = oracle.mixed_attention(x.q, x.k, x.v, alpha, w.softmax_scale, w.sink, w.recent)
        assert_close(got[b], ref, f"mixed-b{B} b{b}")
