"""GPU parity of chunked prefill on layers whose caches are not bf16, against
the oracle, through the C ABI:

* fp16 layers (retrieval cache and ring in fp16, the fp16 MFMA forms of the
  retrieval and streaming kernels);
* 4-bit retrieval caches with an fp16 or a bf16 ring (the chunk is quantised
  on append, then the retrieval kernel dequantises its tiles on the way to
  LDS; the oracle attends over its own fma-dequantised cache);

over ragged chunk lists that span several key tiles and end inside a 32-token
block, with a capacity whose last key tile reaches past the 4-bit block array
(the clamp of the staging loads), decode steps after the prefill (which read
what the prefill cached), the per-sequence prefill of a ragged 4-bit batch,
and the Llama-3-8B GQA head shape at a 4096-token context on sampled rows.
"""
import numpy as np
import pytest
import torch

import oracle
from duo_synth import random_case, round_bf16, round_fp16
from gpu_util import Routed, assert_blocks_close, device, say, to_dev

pytestmark = pytest.mark.gpu

_TDT = {"fp16": torch.float16, "bf16": torch.bfloat16}


def _layer(Hq, Hkv, D, mask, capacity, scale, kv_dtype, retrieval_dtype, S=16, R=64, batch=1):
    import kv_cache_compression_duo_amd as duo
    r = Routed(mask, Hq // Hkv)
    lay = duo.DuoLayer(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, n_retrieval_kv_heads=r.nr,
                       capacity=capacity, softmax_scale=scale, sink=S, recent=R, batch=batch,
                       kv_dtype=kv_dtype, retrieval_dtype=retrieval_dtype, device=device())
    orc = [oracle.OracleLayer(Hq, Hkv, D, mask, scale, S, R, int4=retrieval_dtype == "int4")
           for _ in range(batch)]
    return lay, orc, r


def _case(seed, T, Hq, Hkv, D, kv_dtype):
    kv_round = round_fp16 if kv_dtype == "fp16" else round_bf16
    return random_case(seed, T=T, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, kv_round=kv_round)


def _run(Hq, Hkv, D, mask, chunks, *, kv_dtype, retrieval_dtype, seed, decode_steps=0,
         extra_capacity=0, scale=None, S=16, R=64, sample_rows=None):
    G = Hq // Hkv
    T = sum(chunks)
    scale = D ** -0.5 if scale is None else scale
    label = f"{kv_dtype}/{retrieval_dtype} Hq={Hq} Hkv={Hkv} D={D} chunks={chunks}"
    say(f"case: {label} seed={seed}")
    q, k, v = _case(seed, T + decode_steps, Hq, Hkv, D, kv_dtype)
    tdt = _TDT[kv_dtype]
    lay, (orc,), r = _layer(Hq, Hkv, D, mask, T + decode_steps + extra_capacity, scale,
                            kv_dtype, retrieval_dtype, S, R)
    rq = np.array([mask[h // G] for h in range(Hq)], bool)
    a = 0
    for c in chunks:
        out = lay.prefill_chunk(r.q(to_dev(q[a:a + c]))[None], r.kv(to_dev(k[a:a + c], tdt))[None],
                                r.kv(to_dev(v[a:a + c], tdt))[None])
        rows = None
        if sample_rows is not None and c > sample_rows:
            g = np.random.default_rng(seed + a)
            rows = np.unique(np.concatenate([[0, c - 1], g.choice(c, sample_rows, replace=False)]))
        ref = orc.prefill_chunk(q[a:a + c], k[a:a + c], v[a:a + c], rows=rows)
        got = r.out(out)[0].float().cpu().numpy()
        if rows is not None:
            got, ref = got[rows], ref[rows]
        assert_blocks_close(got, ref, rq, f"{label} chunk@{a}+{c}", head_axis=1)
        a += c
    assert lay.n_tokens == T
    for s in range(decode_steps):
        t = T + s
        out = lay.decode(r.q(to_dev(q[t]))[None, None], r.kv(to_dev(k[t], tdt))[None, None],
                         r.kv(to_dev(v[t], tdt))[None, None])
        ref = orc.decode(q[t], k[t], v[t])
        assert_blocks_close(r.out(out)[0, 0].float().cpu().numpy(), ref, rq,
                            f"{label} decode {s}", head_axis=0)
    return lay, orc


@pytest.mark.parametrize("Hq,Hkv,D,mask", [
    (8, 4, 64, (1, 0, 0, 1)),                 # G = 2, head_dim 64
    (32, 8, 128, (0, 1, 0, 0, 1, 0, 0, 0)),   # G = 4, head_dim 128
    (4, 4, 128, (1, 1, 1, 1)),                # MHA, all retrieval
])
def test_prefill_fp16_layer(Hq, Hkv, D, mask):
    _run(Hq, Hkv, D, mask, [130, 1, 200, 77], kv_dtype="fp16", retrieval_dtype="fp16",
         seed=9400 + Hq + D, decode_steps=3)


@pytest.mark.parametrize("kv_dtype,Hq,Hkv,D,mask", [
    ("fp16", 8, 2, 128, (1, 0)),
    ("bf16", 16, 4, 64, (0, 1, 1, 0)),
    ("fp16", 8, 8, 64, (1, 1, 0, 1, 0, 0, 1, 1)),  # G = 1
    ("bf16", 32, 4, 64, (1, 1, 1, 1)),             # G = 8, all retrieval
])
def test_prefill_int4_layer(kv_dtype, Hq, Hkv, D, mask):
    # 400 prefill tokens + 2 decode steps: capacity 402, 32-token blocks up to
    # 416, while the last prefill key tile covers positions 384..447
    _run(Hq, Hkv, D, mask, [100, 1, 64, 235], kv_dtype=kv_dtype, retrieval_dtype="int4",
         seed=9500 + Hq + D, decode_steps=2)


@pytest.mark.parametrize("chunks", [[1] * 5, [31, 33], [64, 64, 1], [5, 300]])
def test_prefill_int4_chunk_shapes(chunks):
    _run(8, 2, 128, (1, 0), chunks, kv_dtype="fp16", retrieval_dtype="int4",
         seed=9600 + sum(chunks), extra_capacity=7)


def test_prefill_int4_short_window():
    _run(8, 4, 64, (1, 0, 1, 0), [40, 90], kv_dtype="fp16", retrieval_dtype="int4",
         seed=9650, S=3, R=7)


def test_prefill_int4_codes_match_append():
    """Codes a prefill writes equal those of an append of the same rows."""
    Hq, Hkv, D = 8, 2, 128
    q, k, v = _case(9700, 150, Hq, Hkv, D, "fp16")
    layers = []
    for use_prefill in (True, False):
        lay, _, r = _layer(Hq, Hkv, D, (1, 0), 150, D ** -0.5, "fp16", "int4")
        for a, c in ((0, 70), (70, 80)):
            kd = r.kv(to_dev(k[a:a + c], torch.float16))[None]
            vd = r.kv(to_dev(v[a:a + c], torch.float16))[None]
            if use_prefill:
                lay.prefill_chunk(r.q(to_dev(q[a:a + c]))[None], kd, vd)
            else:
                lay.append_kv(kd, vd)
        layers.append(lay)
    torch.cuda.synchronize()
    for x, y in zip(layers[0].retrieval_int4(), layers[1].retrieval_int4()):
        assert torch.equal(x, y)
    say("  4-bit codes and scale/zero words after prefill == after append")


def test_prefill_int4_ragged_sequences():
    """Per-sequence prefill of a batch of 3 whose sequences grow unevenly."""
    Hq, Hkv, D = 16, 4, 128
    mask = (1, 0, 1, 0)
    G = Hq // Hkv
    plan = {0: [70, 130], 1: [1, 33], 2: [257]}
    say(f"case: ragged 4-bit prefill plan={plan}")
    lay, orcs, r = _layer(Hq, Hkv, D, mask, 300, D ** -0.5, "fp16", "int4", batch=3)
    rq = np.array([mask[h // G] for h in range(Hq)], bool)
    data = {b: _case(9800 + b, sum(c), Hq, Hkv, D, "fp16") for b, c in plan.items()}
    pos = {b: 0 for b in plan}
    for step in range(2):
        for b, chunks in plan.items():
            if step >= len(chunks):
                continue
            c, a = chunks[step], pos[b]
            q, k, v = (x[a:a + c] for x in data[b])
            out = lay.prefill_chunk_seq(b, r.q(to_dev(q))[None],
                                        r.kv(to_dev(k, torch.float16))[None],
                                        r.kv(to_dev(v, torch.float16))[None])
            ref = orcs[b].prefill_chunk(q, k, v)
            assert_blocks_close(r.out(out)[0].float().cpu().numpy(), ref, rq,
                                f"seq {b} chunk@{a}+{c}", head_axis=1)
            pos[b] += c
    for b in plan:
        assert lay.sequence_tokens(b) == pos[b]


def test_prefill_int4_llama3_gqa_4k_sampled():
    """Llama-3-8B head shape (32 q / 8 KV heads, 4 retrieval, D = 128): a
    4-bit retrieval cache and fp16 ring over two 2048-token chunks, 64
    sampled query rows per chunk."""
    mask = (1, 0, 1, 1, 0, 0, 1, 0)
    _run(32, 8, 128, mask, [2048, 2048], kv_dtype="fp16", retrieval_dtype="int4", seed=9900,
         sample_rows=64)


@pytest.mark.parametrize("kv_dtype,retrieval_dtype", [("fp16", "int4"), ("bf16", "int4"),
                                                      ("fp16", "fp16")])
def test_prefill_quant_batch2(kv_dtype, retrieval_dtype):
    """Batch-wide prefill of two sequences (each against its own oracle):
    every (sequence, head) finds its own cache rows, codes and scale words."""
    Hq, Hkv, D = 16, 4, 128
    mask = (0, 1, 1, 0)
    G = Hq // Hkv
    chunks = [90, 170]
    say(f"case: batch 2 {kv_dtype}/{retrieval_dtype} chunks={chunks}")
    lay, orcs, r = _layer(Hq, Hkv, D, mask, sum(chunks) + 1, D ** -0.5, kv_dtype,
                          retrieval_dtype, batch=2)
    rq = np.array([mask[h // G] for h in range(Hq)], bool)
    data = [_case(9950 + b, sum(chunks) + 1, Hq, Hkv, D, kv_dtype) for b in range(2)]
    tdt = _TDT[kv_dtype]
    a = 0
    for c in chunks:
        q = torch.stack([r.q(to_dev(data[b][0][a:a + c])) for b in range(2)])
        k = torch.stack([r.kv(to_dev(data[b][1][a:a + c], tdt)) for b in range(2)])
        v = torch.stack([r.kv(to_dev(data[b][2][a:a + c], tdt)) for b in range(2)])
        out = lay.prefill_chunk(q, k, v)
        for b in range(2):
            ref = orcs[b].prefill_chunk(*(x[a:a + c] for x in data[b]))
            assert_blocks_close(r.out(out[b]).float().cpu().numpy(), ref, rq,
                                f"seq {b} chunk@{a}+{c}", head_axis=1)
        a += c
    # one decode step of both sequences after the prefill
    t = a
    out = lay.decode(torch.stack([r.q(to_dev(data[b][0][t]))[None] for b in range(2)]),
                     torch.stack([r.kv(to_dev(data[b][1][t], tdt))[None] for b in range(2)]),
                     torch.stack([r.kv(to_dev(data[b][2][t], tdt))[None] for b in range(2)]))
    for b in range(2):
        ref = orcs[b].decode(*(x[t] for x in data[b]))
        assert_blocks_close(r.out(out[b, 0]).float().cpu().numpy(), ref, rq, f"seq {b} decode",
                            head_axis=0)
