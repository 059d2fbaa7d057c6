"""GPU parity of the matrix-core decode path (layers with four or more query
heads per KV head) against the oracle, through the C ABI.

The path streams 32-row tiles per wave and takes the split-K ranges the host
chooses, so the cases aim at its boundaries: contexts just below, at and
above a 32-row tile and a 256-row split (a split that holds only the new
token appears when the row count is one past a multiple of the split size),
an empty context, a long context whose split size is not a multiple of 32
(split ranges start inside a tile), fp16 caches, head_dim 64 with eight query
heads per KV head, and a ragged batch whose short sequences leave most split
ranges empty.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from duo_synth import WORKLOADS, make_inputs, round_fp16
from gpu_util import Routed, assert_blocks_close, device, say, to_dev

pytestmark = pytest.mark.gpu


def _layer_case(G, D, kv_dtype, Hkv, retrieval, context, steps, seed):
    import kv_cache_compression_duo_amd as duo
    w = dataclasses.replace(WORKLOADS["llama3_8b_prefill_64k"], n_q_heads=G * Hkv, n_kv_heads=Hkv,
                            head_dim=D, fixed_retrieval=retrieval, softmax_scale=D ** -0.5,
                            kv_dtype=kv_dtype, ring_dtype=kv_dtype)
    inp = make_inputs(w, tokens=max(context, 1), steps=steps, seed=seed)
    if kv_dtype == "fp16":  # the oracle sees exactly the values the cache holds
        inp.k, inp.v = round_fp16(inp.k), round_fp16(inp.v)
        inp.k_steps, inp.v_steps = round_fp16(inp.k_steps), round_fp16(inp.v_steps)
    mask = inp.retrieval_mask
    r = Routed(mask, G)
    tdt = torch.bfloat16 if kv_dtype == "bf16" else torch.float16
    lay = duo.DuoLayer(n_q_heads=w.n_q_heads, n_kv_heads=Hkv, head_dim=D,
                       n_retrieval_kv_heads=r.nr, capacity=context + steps,
                       softmax_scale=w.softmax_scale, sink=w.sink, recent=w.recent,
                       kv_dtype=kv_dtype, device=device())
    orc = oracle.OracleLayer(w.n_q_heads, Hkv, D, mask, w.softmax_scale, w.sink, w.recent)
    if context:
        lay.append_kv(r.kv(to_dev(inp.k[:context], tdt))[None],
                      r.kv(to_dev(inp.v[:context], tdt))[None])
        orc.append(inp.k[:context], inp.v[:context])
    rq = np.array([mask[h // G] for h in range(w.n_q_heads)], bool)
    for s in range(steps):
        out = lay.decode(r.q(to_dev(inp.q_steps[s]))[None, None],
                         r.kv(to_dev(inp.k_steps[s], tdt))[None, None],
                         r.kv(to_dev(inp.v_steps[s], tdt))[None, None])
        ref = orc.decode(inp.q_steps[s], inp.k_steps[s], inp.v_steps[s])
        assert_blocks_close(r.out(out)[0, 0].float().cpu().numpy(), ref, rq,
                            f"G{G} D{D} {kv_dtype} ctx {context} step {s}", head_axis=0)
    assert lay.n_tokens == context + steps


@pytest.mark.parametrize("context", [0, 1, 31, 32, 33, 127, 128, 129, 255, 256, 257, 511, 512,
                                     1000])
def test_mma_decode_tile_and_split_boundaries(context):
    say(f"case: matrix-core decode G=4 D=128 bf16, context {context} + 2 steps")
    _layer_case(4, 128, "bf16", 4, (0, 3), context, 2, 31000 + context)


@pytest.mark.parametrize("G,D,kv_dtype,context", [(4, 128, "fp16", 777), (8, 64, "bf16", 545),
                                                  (8, 128, "fp16", 300), (4, 64, "fp16", 1029)])
def test_mma_decode_shapes(G, D, kv_dtype, context):
    say(f"case: matrix-core decode G={G} D={D} {kv_dtype}, context {context} + 3 steps")
    _layer_case(G, D, kv_dtype, 2, (1,), context, 3, 31500 + G * D + context)


def test_mma_decode_long_context_unaligned_splits():
    """One retrieval KV head at a 60000-token context: the split size (the rows
    over the blocks a head gets) is not a multiple of the 32-row tile."""
    say("case: matrix-core decode G=4 D=128 bf16, context 60000 + 2 steps")
    _layer_case(4, 128, "bf16", 2, (0,), 60000, 2, 31900)


def test_mma_decode_ragged_batch():
    """Four sequences of a G = 4 layer at very different lengths decoded
    together, each against its own oracle layer."""
    import kv_cache_compression_duo_amd as duo
    w = dataclasses.replace(WORKLOADS["llama3_8b_prefill_64k"], n_q_heads=16, n_kv_heads=4,
                            fixed_retrieval=(0, 2))
    contexts, steps = (2000, 1, 33, 256), 3
    say(f"case: matrix-core ragged decode, contexts {contexts}")
    inps = [make_inputs(w, tokens=contexts[b], steps=steps, seed=32000 + 7 * b)
            for b in range(len(contexts))]
    mask = inps[0].retrieval_mask
    G = 4
    r = Routed(mask, G)
    lay = duo.DuoLayer(n_q_heads=16, n_kv_heads=4, head_dim=128, n_retrieval_kv_heads=r.nr,
                       capacity=max(contexts) + steps, softmax_scale=w.softmax_scale,
                       sink=w.sink, recent=w.recent, batch=len(contexts), device=device())
    orcs = [oracle.OracleLayer(16, 4, 128, mask, w.softmax_scale, w.sink, w.recent)
            for _ in contexts]
    for b, (x, o) in enumerate(zip(inps, orcs)):
        lay.append_kv_seq(b, r.kv(to_dev(x.k, torch.bfloat16))[None],
                          r.kv(to_dev(x.v, torch.bfloat16))[None])
        o.append(x.k, x.v)
    rq = np.array([mask[h // G] for h in range(16)], bool)
    for s in range(steps):
        q = torch.stack([r.q(to_dev(x.q_steps[s]))[None] for x in inps]).contiguous()
        k = torch.stack([r.kv(to_dev(x.k_steps[s], torch.bfloat16))[None] for x in inps])
        v = torch.stack([r.kv(to_dev(x.v_steps[s], torch.bfloat16))[None] for x in inps])
        got = r.out(lay.decode(q, k.contiguous(), v.contiguous())).float().cpu().numpy()
        for b, (x, o) in enumerate(zip(inps, orcs)):
            ref = o.decode(x.q_steps[s], x.k_steps[s], x.v_steps[s])
            assert_blocks_close(got[b, 0], ref, rq, f"ragged step {s} b{b}", head_axis=0)
    assert [lay.sequence_tokens(b) for b in range(len(contexts))] == [c + steps for c in contexts]
