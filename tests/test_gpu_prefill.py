"""GPU parity of chunked prefill (retrieval MFMA kernel + streaming Lambda
kernel + cache/ring appends) against the oracle, through the C ABI.

Covers: the 8-head D=64 layer (prefill 1024 as one chunk, then 16 decode
steps); the Llama-3-8B GQA layer (32q/8kv, 4 retrieval KV heads by seed) over
several ragged chunks and at its full 65536-token / 8192-chunk size on sampled
rows; chunk sizes that are not tile multiples; sequences shorter than the
sink, around S + R; group sizes 1, 2, 4, 8; head_dim 64/128; all-streaming
and all-retrieval layers; chunked vs one-shot equality.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from duo_synth import WORKLOADS, make_inputs, round_bf16
from gpu_util import Routed, assert_blocks_close, device, say, to_dev

pytestmark = pytest.mark.gpu


def _layer(inp, capacity, batch=1):
    import kv_cache_compression_duo_amd as duo
    w = inp.workload
    Hq = w.n_q_heads
    r = Routed(inp.retrieval_mask, Hq // w.n_kv_heads)
    lay = duo.DuoLayer(n_q_heads=Hq, n_kv_heads=w.n_kv_heads, head_dim=w.head_dim,
                       n_retrieval_kv_heads=r.nr, capacity=capacity,
                       softmax_scale=w.softmax_scale, sink=w.sink, recent=w.recent,
                       batch=batch, device=device())
    orc = oracle.OracleLayer(Hq, w.n_kv_heads, w.head_dim, inp.retrieval_mask,
                             w.softmax_scale, w.sink, w.recent)
    return lay, orc, r


def _run_prefill(inp, chunks, *, decode_steps=0, sample_rows=None, label=""):
    """Prefill inp.q/k/v in the given chunk lengths (then decode), comparing
    every chunk (or `sample_rows` rows per chunk) with the oracle."""
    w = inp.workload
    T = sum(chunks)
    G = w.n_q_heads // w.n_kv_heads
    lay, orc, r = _layer(inp, T + decode_steps)
    rq = np.array([inp.retrieval_mask[h // G] for h in range(w.n_q_heads)], bool)
    a = 0
    for c in chunks:
        q, k, v = inp.q[a:a + c], inp.k[a:a + c], inp.v[a:a + c]
        out = lay.prefill_chunk(r.q(to_dev(q))[None], r.kv(to_dev(k))[None], r.kv(to_dev(v))[None])
        rows = None
        if sample_rows is not None and c > sample_rows:
            g = np.random.default_rng(a)
            rows = np.unique(np.concatenate([[0, c - 1], g.choice(c, sample_rows, replace=False)]))
        ref = orc.prefill_chunk(q, k, v, rows=rows)
        got = r.out(out)[0].float().cpu().numpy()
        if rows is not None:
            got, ref = got[rows], ref[rows]
        assert_blocks_close(got, ref, rq, f"{label} chunk@{a}+{c}", head_axis=1)
        a += c
    assert lay.n_tokens == T
    for s in range(decode_steps):
        out = lay.decode(r.q(to_dev(inp.q_steps[s]))[None, None],
                         r.kv(to_dev(inp.k_steps[s]))[None, None],
                         r.kv(to_dev(inp.v_steps[s]))[None, None])
        ref = orc.decode(inp.q_steps[s], inp.k_steps[s], inp.v_steps[s])
        assert_blocks_close(r.out(out)[0, 0].float().cpu().numpy(), ref, rq,
                            f"{label} decode {s}", head_axis=0)
    return lay, orc, r


def test_prefill_mha8_d64_then_decode():
    w = WORKLOADS["mha8_d64_seq1024"]
    say(f"case: {w.key} prefill 1024 + 16 decode")
    inp = make_inputs(w)
    _run_prefill(inp, [1024], decode_steps=16, label=w.key)


def test_prefill_llama3_gqa_ragged_chunks():
    w = WORKLOADS["llama3_8b_prefill_64k"]
    say(f"case: {w.key} 2500 tokens in chunks 1000/1000/500")
    inp = make_inputs(w, tokens=2500)
    _run_prefill(inp, [1000, 1000, 500], label=w.key)


def test_prefill_llama3_gqa_full_size_sampled():
    w = WORKLOADS["llama3_8b_prefill_64k"]
    say(f"case: {w.key} 65536 tokens in 8 x 8192 chunks, sampled rows")
    inp = make_inputs(w)
    _run_prefill(inp, [8192] * 8, sample_rows=24, label=w.key)


@pytest.mark.parametrize("chunks", [[1] * 9, [7, 7, 7], [33, 64, 65], [127, 129, 1], [300]])
def test_prefill_chunk_shapes(chunks):
    w = dataclasses.replace(WORKLOADS["llama3_8b_prefill_64k"], n_q_heads=8, n_kv_heads=2,
                            fixed_retrieval=(1,))
    say(f"case: chunks {chunks}")
    inp = make_inputs(w, tokens=sum(chunks), seed=6000 + len(chunks))
    _run_prefill(inp, chunks, label=f"chunks{chunks}")


@pytest.mark.parametrize("T", [5, 16, 79, 80, 81, 200])
def test_prefill_around_sink_and_window(T):
    w = dataclasses.replace(WORKLOADS["mha8_d64_seq1024"], n_q_heads=4, n_kv_heads=4,
                            fixed_retrieval=(2,))
    say(f"case: one chunk of {T}, then 3 decode steps")
    inp = make_inputs(w, tokens=T, steps=3, seed=7000 + T)
    _run_prefill(inp, [T], decode_steps=3, label=f"T{T}")


@pytest.mark.parametrize("S,R", [(0, 5), (0, 9), (3, 7)])
def test_prefill_short_window_no_sink(S, R):
    # without sink tokens a block's first Lambda tile is a window tile, and
    # rows of its later waves have no key in it
    w = dataclasses.replace(WORKLOADS["mha8_d64_seq1024"], n_q_heads=4, n_kv_heads=4,
                            fixed_retrieval=(2,), sink=S, recent=R)
    say(f"case: S={S} R={R}, chunks 130/170, then 2 decode steps")
    inp = make_inputs(w, tokens=300, steps=2, seed=7100 + 10 * S + R)
    _run_prefill(inp, [130, 170], decode_steps=2, label=f"S{S}R{R}")


def test_prefill_rising_scores_rescale():
    # key norms rising 1x -> 3x along the sequence: each query's scores grow
    # tile after tile, so the running softmax reference moves up many times
    # (the rescale path of the retrieval and streaming loops), from a first
    # tile whose reference is taken fresh
    w = dataclasses.replace(WORKLOADS["llama3_8b_prefill_64k"], n_q_heads=8, n_kv_heads=2,
                            fixed_retrieval=(1,))
    say("case: 640 tokens, key norms rising 1x..3x, chunks 256/384")
    inp = make_inputs(w, tokens=640, seed=9100)
    ramp = (1.0 + 2.0 * np.arange(640) / 640)[:, None, None]
    inp.k = round_bf16(inp.k * ramp)
    _run_prefill(inp, [256, 384], label="rising")


def test_prefill_large_logits_exact_scale(monkeypatch):
    # queries doubled and key norms rising 1x..3x: exp2 arguments spread over
    # about 7 per query, where rounding q * scale * log2(e) to bf16 moves the
    # outputs past the bar (max-abs about 0.027 in a float64 simulation);
    # DUO_EXACT_SCALE=1 selects the form that applies the scale in fp32
    monkeypatch.setenv("DUO_EXACT_SCALE", "1")
    w = dataclasses.replace(WORKLOADS["llama3_8b_prefill_64k"], n_q_heads=8, n_kv_heads=2,
                            fixed_retrieval=(1,))
    say("case: 640 tokens, q x2, key norms rising 1x..3x, exact scale, chunks 256/384")
    inp = make_inputs(w, tokens=640, seed=9100)
    ramp = (1.0 + 2.0 * np.arange(640) / 640)[:, None, None]
    inp.k = round_bf16(inp.k * ramp)
    inp.q = round_bf16(inp.q * 2.0)
    _run_prefill(inp, [256, 384], label="large logits, exact scale")


@pytest.mark.parametrize("G,D", [(1, 128), (2, 64), (4, 64), (8, 128)])
def test_prefill_group_sizes(G, D):
    w = dataclasses.replace(WORKLOADS["llama3_8b_prefill_64k"], n_q_heads=2 * G, n_kv_heads=2,
                            head_dim=D, fixed_retrieval=(0,), softmax_scale=D ** -0.5)
    say(f"case: G={G} D={D}")
    inp = make_inputs(w, tokens=400, seed=8000 + G * 10 + D)
    _run_prefill(inp, [150, 250], label=f"G{G}D{D}")


@pytest.mark.parametrize("heads", [(), (0, 1, 2)])
def test_prefill_all_streaming_or_all_retrieval(heads):
    w = dataclasses.replace(WORKLOADS["mha8_d64_seq1024"], n_q_heads=3, n_kv_heads=3,
                            fixed_retrieval=heads)
    say(f"case: retrieval heads {heads}")
    inp = make_inputs(w, tokens=500, steps=2, seed=9000 + len(heads))
    _run_prefill(inp, [200, 300], decode_steps=2, label=f"hr{len(heads)}")


@pytest.mark.parametrize("S,R", [(0, 1), (2, 3), (100, 20)])
def test_prefill_other_windows(S, R):
    w = dataclasses.replace(WORKLOADS["mha8_d64_seq1024"], n_q_heads=4, n_kv_heads=2,
                            fixed_retrieval=(0,), sink=S, recent=R)
    say(f"case: window S={S} R={R}")
    inp = make_inputs(w, tokens=330, seed=9100 + S + R)
    _run_prefill(inp, [130, 200], label=f"S{S}R{R}")


def test_chunked_equals_one_shot_on_gpu():
    w = dataclasses.replace(WORKLOADS["llama3_8b_prefill_64k"], n_q_heads=8, n_kv_heads=2,
                            fixed_retrieval=(0,))
    inp = make_inputs(w, tokens=700, seed=9200)
    outs = []
    for chunks in ([700], [100, 250, 350]):
        lay, orc, r = _layer(inp, 700)
        parts = []
        a = 0
        for c in chunks:
            parts.append(lay.prefill_chunk(r.q(to_dev(inp.q[a:a + c]))[None],
                                           r.kv(to_dev(inp.k[a:a + c]))[None],
                                           r.kv(to_dev(inp.v[a:a + c]))[None]).float().cpu())
            a += c
        outs.append(torch.cat(parts, dim=1))
    d = (outs[0] - outs[1]).abs().max().item()
    say(f"  chunked vs one-shot max diff {d:.3e}")
    assert d <= 2e-2
