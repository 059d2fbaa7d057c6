"""GPU parity of the gate-blended mixed forward (head identification form)
against the oracle: the Llama-2-7B 32x128 layer at a ragged length and at its
full 16384-token length on sampled rows, alpha = 1 (full) and alpha = 0
(streaming), GQA, head_dim 64, lengths around the sink/window sizes."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from duo_synth import WORKLOADS, make_inputs, rng
from gpu_util import assert_close, device, say, to_dev

pytestmark = pytest.mark.gpu


def _mixed(inp, alpha, rows=None, label=""):
    import kv_cache_compression_duo_amd as duo
    w = inp.workload
    dev = device()
    q, k, v = to_dev(inp.q)[None], to_dev(inp.k)[None], to_dev(inp.v)[None]
    a = torch.from_numpy(np.asarray(alpha, np.float32)).to(dev)
    out = duo.mixed_forward(q, k, v, a, softmax_scale=w.softmax_scale, sink=w.sink,
                            recent=w.recent)
    got = out[0].float().cpu().numpy()
    ref = oracle.mixed_attention(inp.q, inp.k, inp.v, alpha, w.softmax_scale, w.sink, w.recent,
                                 rows=rows)
    if rows is not None:
        got, ref = got[rows], ref[rows]
    assert_close(got, ref, label)
    return got


def test_mixed_llama2_ragged():
    w = WORKLOADS["llama2_7b_mixed_16k"]
    say(f"case: {w.key} T=1500")
    inp = make_inputs(w, tokens=1500)
    _mixed(inp, inp.alpha, label=w.key)


def test_mixed_llama2_ragged_exact_scale(monkeypatch):
    # the fp32-scale form of the gate-blended forward (DUO_EXACT_SCALE=1)
    monkeypatch.setenv("DUO_EXACT_SCALE", "1")
    test_mixed_llama2_ragged()


def test_mixed_llama2_full_length_sampled():
    w = WORKLOADS["llama2_7b_mixed_16k"]
    say(f"case: {w.key} T=16384, sampled rows")
    inp = make_inputs(w)
    g = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 79, 80, 16383], g.choice(16384, 40, replace=False)]))
    _mixed(inp, inp.alpha, rows=rows, label=w.key)


@pytest.mark.parametrize("alpha_value", [0.0, 1.0])
def test_mixed_alpha_extremes(alpha_value):
    w = dataclasses.replace(WORKLOADS["llama2_7b_mixed_16k"], n_q_heads=4, n_kv_heads=4)
    say(f"case: alpha = {alpha_value}")
    inp = make_inputs(w, tokens=600, seed=9300)
    alpha = np.full(4, alpha_value, np.float32)
    got = _mixed(inp, alpha, label=f"alpha{alpha_value}")
    kind = oracle.full_attention if alpha_value == 1.0 else oracle.streaming_attention
    if alpha_value == 1.0:
        ref = oracle.full_attention(inp.q, inp.k, inp.v, w.softmax_scale)
    else:
        ref = oracle.streaming_attention(inp.q, inp.k, inp.v, w.softmax_scale, w.sink, w.recent)
    assert_close(got, ref, f"alpha{alpha_value} vs plain")


@pytest.mark.parametrize("G,D,T", [(4, 128, 333), (2, 64, 80), (1, 64, 81), (8, 64, 17), (1, 128, 1)])
def test_mixed_shapes(G, D, T):
    w = dataclasses.replace(WORKLOADS["llama2_7b_mixed_16k"], n_q_heads=2 * G, n_kv_heads=2,
                            head_dim=D, softmax_scale=D ** -0.5)
    say(f"case: mixed G={G} D={D} T={T}")
    inp = make_inputs(w, tokens=T, seed=9400 + T)
    _mixed(inp, inp.alpha, label=f"G{G}D{D}T{T}")


@pytest.mark.parametrize("S,R", [(0, 1), (0, 5), (3, 7)])
def test_mixed_short_window_no_sink(S, R):
    # no sink tokens / short windows: Lambda-phase rows of a block's later
    # waves have no allowed key in its first visited tile
    w = dataclasses.replace(WORKLOADS["llama2_7b_mixed_16k"], n_q_heads=4, n_kv_heads=4, sink=S,
                            recent=R)
    say(f"case: mixed S={S} R={R} T=200")
    inp = make_inputs(w, tokens=200, seed=9600 + 10 * S + R)
    _mixed(inp, inp.alpha, label=f"S{S}R{R}")
