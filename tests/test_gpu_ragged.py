"""GPU parity of ragged batches: sequences of one layer holding different
token counts, filled one sequence at a time (duo_append_kv_seq /
duo_prefill_chunk_seq) and decoded together, every sequence at its own
position (duo_decode), through the C ABI. Each sequence is compared with an
oracle layer that sees only that sequence's inputs. Covers the bf16 and fp16
caches, the 4-bit cache, chunked prefill per sequence, a very short sequence
beside a long one (most of its split-K ranges hold no row), sequences
catching up to equal counts, and the batch-wide calls refusing a ragged
layer."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from duo_synth import WORKLOADS, make_inputs, round_fp16
from gpu_util import Routed, assert_blocks_close, device, say, to_dev

pytestmark = pytest.mark.gpu


def _setup(w, B, contexts, steps, seed, kv_dtype="bf16", retrieval_dtype=None, int4=False):
    import kv_cache_compression_duo_amd as duo
    inps = [make_inputs(w, tokens=contexts[b], steps=steps, seed=seed + 101 * b)
            for b in range(B)]
    mask = inps[0].retrieval_mask
    assert all((x.retrieval_mask == mask).all() for x in inps)
    if kv_dtype == "fp16":  # the oracle sees exactly the values the cache holds
        for x in inps:
            x.k, x.v = round_fp16(x.k), round_fp16(x.v)
            x.k_steps, x.v_steps = round_fp16(x.k_steps), round_fp16(x.v_steps)
    G = w.n_q_heads // w.n_kv_heads
    r = Routed(mask, G)
    kw = {} if retrieval_dtype is None else {"retrieval_dtype": retrieval_dtype}
    lay = duo.DuoLayer(n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                       n_retrieval_kv_heads=r.nr, capacity=max(contexts) + steps + 64,
                       softmax_scale=w.softmax_scale, sink=w.sink, recent=w.recent, batch=B,
                       kv_dtype=kv_dtype, device=device(), **kw)
    orcs = [oracle.OracleLayer(w.n_q_heads, w.n_kv_heads, w.head_dim, mask, w.softmax_scale,
                               w.sink, w.recent, int4=int4) for _ in range(B)]
    rq = np.array([mask[h // G] for h in range(w.n_q_heads)], bool)
    return inps, lay, orcs, r, rq


def _decode(lay, r, inps, orcs, steps, dtype, rq, label, first=0):
    for s in range(first, first + steps):
        q = torch.stack([r.q(to_dev(x.q_steps[s]))[None] for x in inps]).contiguous()
        k = torch.stack([r.kv(to_dev(x.k_steps[s], dtype))[None] for x in inps]).contiguous()
        v = torch.stack([r.kv(to_dev(x.v_steps[s], dtype))[None] for x in inps]).contiguous()
        got = r.out(lay.decode(q, k, v)).float().cpu().numpy()
        for b, (x, o) in enumerate(zip(inps, orcs)):
            ref = o.decode(x.q_steps[s], x.k_steps[s], x.v_steps[s])
            assert_blocks_close(got[b, 0], ref, rq, f"{label} step {s} b{b}", head_axis=0)


@pytest.mark.parametrize("kv_dtype,contexts", [("bf16", (300, 137, 64)),
                                               ("fp16", (900, 3, 81)),
                                               ("bf16", (3000, 5))])
def test_ragged_decode(kv_dtype, contexts):
    w = dataclasses.replace(WORKLOADS["llama3_8b_prefill_64k"], n_q_heads=8, n_kv_heads=4,
                            fixed_retrieval=(0, 2))
    B, steps = len(contexts), 3
    dtype = torch.bfloat16 if kv_dtype == "bf16" else torch.float16
    say(f"case: ragged decode {kv_dtype}, contexts {contexts}")
    inps, lay, orcs, r, rq = _setup(w, B, contexts, steps, 22000 + sum(contexts), kv_dtype)
    for b, (x, o) in enumerate(zip(inps, orcs)):
        lay.append_kv_seq(b, r.kv(to_dev(x.k, dtype))[None], r.kv(to_dev(x.v, dtype))[None])
        o.append(x.k, x.v)
    assert [lay.sequence_tokens(b) for b in range(B)] == list(contexts)
    assert lay.n_tokens == max(contexts)
    _decode(lay, r, inps, orcs, steps, dtype, rq, f"ragged-{kv_dtype}")
    assert [lay.sequence_tokens(b) for b in range(B)] == [c + steps for c in contexts]


@pytest.mark.parametrize("retrieval_dtype", [None, "int4"])
def test_ragged_decode_more_sequences_than_one_launch_takes(retrieval_dtype):
    """70 sequences of different lengths: the decode runs in slices of 64
    sequences, one launch each, sharing the workspace."""
    int4 = retrieval_dtype == "int4"
    base = WORKLOADS["llama3_8b_int4_decode_1m" if int4 else "mha8_d64_seq1024"]
    w = dataclasses.replace(base, n_q_heads=4, n_kv_heads=2, fixed_retrieval=(1,))
    g = np.random.default_rng(26000)
    contexts = tuple(int(x) for x in g.integers(1, 200, size=70))
    steps = 2
    kv = "fp16" if int4 else "bf16"
    say(f"case: ragged decode of 70 sequences ({retrieval_dtype or kv} retrieval cache)")
    inps, lay, orcs, r, rq = _setup(w, 70, contexts, steps, 26000, kv_dtype=kv,
                                    retrieval_dtype=retrieval_dtype, int4=int4)
    dtype = torch.float16 if int4 else torch.bfloat16
    for b, (x, o) in enumerate(zip(inps, orcs)):
        lay.append_kv_seq(b, r.kv(to_dev(x.k, dtype))[None], r.kv(to_dev(x.v, dtype))[None])
        o.append(x.k, x.v)
    _decode(lay, r, inps, orcs, steps, dtype, rq, f"ragged70-{retrieval_dtype or kv}")
    assert [lay.sequence_tokens(b) for b in range(70)] == [c + steps for c in contexts]


def test_ragged_int4_decode():
    w = dataclasses.replace(WORKLOADS["llama3_8b_int4_decode_1m"], fixed_retrieval=(0, 3, 5, 6))
    contexts, steps = (700, 45), 3
    say(f"case: ragged 4-bit decode, contexts {contexts}")
    inps, lay, orcs, r, rq = _setup(w, 2, contexts, steps, 23000, kv_dtype="fp16",
                                    retrieval_dtype="int4", int4=True)
    for b, (x, o) in enumerate(zip(inps, orcs)):
        lay.append_kv_seq(b, r.kv(to_dev(x.k, torch.float16))[None],
                          r.kv(to_dev(x.v, torch.float16))[None])
        o.append(x.k, x.v)
    _decode(lay, r, inps, orcs, steps, torch.float16, rq, "ragged-int4")


def test_prefill_per_sequence_then_decode():
    w = dataclasses.replace(WORKLOADS["llama3_8b_prefill_64k"], n_q_heads=16, n_kv_heads=4,
                            fixed_retrieval=(1, 2))
    chunks = ([100, 77], [50])
    steps = 2
    say(f"case: prefill per sequence, chunks {chunks}, then {steps} decode steps")
    inps, lay, orcs, r, rq = _setup(w, 2, [sum(c) for c in chunks], steps, 24000)
    for b, (x, o) in enumerate(zip(inps, orcs)):
        a = 0
        for c in chunks[b]:
            got = lay.prefill_chunk_seq(b, r.q(to_dev(x.q[a:a + c]))[None],
                                        r.kv(to_dev(x.k[a:a + c]))[None],
                                        r.kv(to_dev(x.v[a:a + c]))[None])
            ref = o.prefill_chunk(x.q[a:a + c], x.k[a:a + c], x.v[a:a + c])
            assert_blocks_close(r.out(got)[0].float().cpu().numpy(), ref, rq,
                                f"seq {b} chunk@{a}+{c}", head_axis=1)
            a += c
    _decode(lay, r, inps, orcs, steps, torch.bfloat16, rq, "prefill-seq decode")


def test_batch_calls_refuse_ragged_and_resume_when_equal():
    import kv_cache_compression_duo_amd as duo
    w = dataclasses.replace(WORKLOADS["llama3_8b_prefill_64k"], n_q_heads=4, n_kv_heads=2,
                            fixed_retrieval=(0,))
    say("case: batch-wide calls on a ragged layer")
    inps, lay, orcs, r, rq = _setup(w, 2, (40, 40), 2, 25000)
    x0, x1 = inps
    lay.append_kv_seq(0, r.kv(to_dev(x0.k[:30]))[None], r.kv(to_dev(x0.v[:30]))[None])
    lay.append_kv_seq(1, r.kv(to_dev(x1.k[:20]))[None], r.kv(to_dev(x1.v[:20]))[None])
    k = torch.stack([r.kv(to_dev(x.k[30:40]))[None][0] for x in inps]).contiguous()
    with pytest.raises(duo.DuoError) as e:
        lay.append_kv(k, k)
    assert e.value.status == 2
    with pytest.raises(duo.DuoError) as e:
        lay.append_kv_seq(2, k[:1], k[:1])
    assert e.value.status == 1
    # sequence 1 catches up: the batch-wide calls work again
    lay.append_kv_seq(1, r.kv(to_dev(x1.k[20:30]))[None], r.kv(to_dev(x1.v[20:30]))[None])
    lay.append_kv(k, torch.stack([r.kv(to_dev(x.v[30:40]))[None][0] for x in inps]).contiguous())
    for x, o in zip(inps, orcs):
        o.append(x.k, x.v)
    assert lay.n_tokens == 40 and lay.sequence_tokens(1) == 40
    _decode(lay, r, inps, orcs, 2, torch.bfloat16, rq, "caught-up")



@pytest.mark.parametrize("retrieval_dtype", [None, "int4"])
def test_ragged_slices_with_many_retrieval_heads_then_batch_wide(retrieval_dtype):
    """70 ragged sequences with 8 retrieval KV heads decode in two launches
    per step (64 + 6 sequences); then every sequence catches up to the same
    count and the batch-wide launch runs. All three launch shapes must find
    the split-K arrival counters and partials at the same workspace offsets
    (laid out for the whole batch): a counter overwritten by another launch's
    partials would leave some head's output unwritten."""
    int4 = retrieval_dtype == "int4"
    base = WORKLOADS["llama3_8b_int4_decode_1m" if int4 else "llama2_7b_decode_32k"]
    # 12 KV heads of which 8 are retrieval heads; the 4-bit decode maps
    # G * D / 32 <= 16 columns, G = 2 here
    w = dataclasses.replace(base, n_q_heads=24 if int4 else 12, n_kv_heads=12, head_dim=128,
                            fixed_retrieval=(0, 1, 2, 4, 5, 7, 9, 11))
    B, steps = 70, 2
    g = np.random.default_rng(27000)
    contexts = [int(x) for x in g.integers(1, 160, size=B)]
    common = max(contexts) + steps + 1  # count every sequence reaches before phase 2
    kv = "fp16" if int4 else "bf16"
    dtype = torch.float16 if int4 else torch.bfloat16
    say(f"case: 70 ragged sequences, 8 retrieval heads, sliced then batch-wide "
        f"({retrieval_dtype or kv} retrieval cache)")
    inps, lay, orcs, r, rq = _setup(w, B, [common - steps] * B, 2 * steps, 27000, kv_dtype=kv,
                                    retrieval_dtype=retrieval_dtype, int4=int4)
    assert r.nr == 8
    for b, (x, o) in enumerate(zip(inps, orcs)):
        c = contexts[b]
        lay.append_kv_seq(b, r.kv(to_dev(x.k[:c], dtype))[None], r.kv(to_dev(x.v[:c], dtype))[None])
        o.append(x.k[:c], x.v[:c])
    _decode(lay, r, inps, orcs, steps, dtype, rq, "ragged70x8 sliced")
    for b, (x, o) in enumerate(zip(inps, orcs)):
        c = contexts[b]
        lay.append_kv_seq(b, r.kv(to_dev(x.k[c:common - steps], dtype))[None],
                          r.kv(to_dev(x.v[c:common - steps], dtype))[None])
        o.append(x.k[c:common - steps], x.v[c:common - steps])
    assert [lay.sequence_tokens(b) for b in range(B)] == [common] * B
    _decode(lay, r, inps, orcs, steps, dtype, rq, "ragged70x8 batch-wide", first=steps)
    assert [lay.sequence_tokens(b) for b in range(B)] == [common + steps] * B
