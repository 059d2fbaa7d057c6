"""GPU parity of the block-sparse Lambda mask (64-token blocks, the form used
while training the gates) in the gate-blended forward and its gate gradient,
through the C ABI (duo_mixed_forward_block, duo_mixed_alpha_grad_block),
against the oracle's block mask: several sink / window sizes (one or several
sink blocks, one to three local blocks, no sinks), GQA and head_dim 64,
ragged lengths, alpha = 0 (the block-streaming attention alone), and the
16384-token Llama-2-7B identification layer on sampled rows. The forward
uses the output bar; the gradient the derived bound of gpu_util."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from duo_synth import WORKLOADS, make_inputs, normal, random_case, rng, round_bf16
from gpu_util import assert_close, device, grad_tolerance, say, to_dev

pytestmark = pytest.mark.gpu

BLOCK = 64


def _forward(q, k, v, alpha, scale, S, R):
    import kv_cache_compression_duo_amd as duo
    dev = device()
    a = torch.from_numpy(np.asarray(alpha, np.float32)).to(dev)
    out = duo.mixed_forward(to_dev(q)[None], to_dev(k)[None], to_dev(v)[None], a,
                            softmax_scale=scale, sink=S, recent=R, lambda_block=BLOCK)
    return out[0].float().cpu().numpy()


@pytest.mark.parametrize("T,Hq,Hkv,D,S,R", [
    (333, 8, 4, 128, 16, 64),    # one sink block, one local block
    (700, 4, 4, 64, 100, 130),   # two sink blocks, three local blocks
    (260, 8, 2, 128, 0, 64),     # no sinks
    (129, 16, 2, 128, 64, 65),   # block-aligned sinks, two local blocks
    (300, 16, 2, 64, 16, 64),    # G=8, head_dim 64
])
def test_block_mixed_forward_matches_oracle(T, Hq, Hkv, D, S, R):
    scale = D ** -0.5
    q, k, v = random_case(20000 + T + S, T=T, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D)
    alpha = np.linspace(0.0, 1.0, Hkv).astype(np.float32)
    say(f"case: block-sparse mixed T={T} Hq={Hq} Hkv={Hkv} D={D} S={S} R={R}")
    got = _forward(q, k, v, alpha, scale, S, R)
    ref = oracle.mixed_attention(q, k, v, alpha, scale, S, R, block=BLOCK)
    assert_close(got, ref, f"block mixed T{T} S{S} R{R}")


def test_block_streaming_alone():
    T, H, D, S, R = 500, 4, 128, 16, 64
    q, k, v = random_case(20500, T=T, n_q_heads=H, n_kv_heads=H, head_dim=D)
    say("case: block-sparse streaming attention alone (alpha = 0)")
    got = _forward(q, k, v, np.zeros(H, np.float32), D ** -0.5, S, R)
    ref = np.stack([oracle.masked_attention(q[:, h], k[:, h], v[:, h], np.arange(T), np.arange(T),
                                            D ** -0.5, "streaming", S, R, block=BLOCK)
                    for h in range(H)], axis=1)
    assert_close(got, ref, "block streaming")
    # the token-level mask differs from the block mask here
    tok = oracle.streaming_attention(q, k, v, D ** -0.5, S, R)
    assert np.abs(tok - ref).max() > 0.05


def test_block_mixed_full_length_sampled():
    w = WORKLOADS["llama2_7b_mixed_16k"]
    say(f"case: {w.key} T=16384 block-sparse, sampled rows")
    inp = make_inputs(w)
    g = np.random.default_rng(7)
    rows = np.unique(np.concatenate([[0, 63, 64, 127, 128, 16383],
                                     g.choice(16384, 30, replace=False)]))
    got = _forward(inp.q, inp.k, inp.v, inp.alpha, w.softmax_scale, w.sink, w.recent)
    ref = oracle.mixed_attention(inp.q, inp.k, inp.v, inp.alpha, w.softmax_scale, w.sink,
                                 w.recent, rows=rows, block=BLOCK)
    assert_close(got[rows], ref[rows], f"{w.key} block sampled")


@pytest.mark.parametrize("T,Hq,Hkv,D,S,R", [
    (333, 8, 4, 128, 16, 64),
    (400, 4, 2, 64, 100, 130),
    (200, 16, 2, 64, 16, 64),    # G=8, head_dim 64
])
def test_block_alpha_grad_matches_oracle(T, Hq, Hkv, D, S, R):
    import kv_cache_compression_duo_amd as duo
    dev = device()
    scale, l1 = D ** -0.5, 0.05
    q, k, v = random_case(21000 + T, T=T, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D)
    dout = round_bf16(normal(rng(21001 + T), (T, Hq, D)))
    alpha = np.linspace(-0.5, 1.0, Hkv).astype(np.float32)
    say(f"case: block-sparse alpha grad T={T} Hq={Hq} Hkv={Hkv} D={D} S={S} R={R}")
    g = duo.mixed_alpha_grad(to_dev(q)[None], to_dev(k)[None], to_dev(v)[None],
                             to_dev(dout)[None], torch.from_numpy(alpha).to(dev),
                             softmax_scale=scale, sink=S, recent=R, l1_weight=l1,
                             lambda_block=BLOCK)
    got = g.cpu().numpy().astype(np.float64)
    ref = oracle.mixed_alpha_grad(q, k, v, dout, alpha, scale, S, R, l1_weight=l1, block=BLOCK)
    tol = grad_tolerance(q, k, v, dout, scale, S, R, block=BLOCK)
    say(f"  max |got - ref| = {np.abs(got - ref).max():.3e}, min tolerance {tol.min():.3e}")
    assert np.all(np.abs(got - ref) <= tol), (got, ref, tol)


def test_block_rejects_other_block_sizes():
    import kv_cache_compression_duo_amd as duo
    dev = device()
    q = torch.zeros(1, 64, 4, 64, dtype=torch.bfloat16, device=dev)
    kv = torch.zeros(1, 64, 4, 64, dtype=torch.bfloat16, device=dev)
    a = torch.zeros(4, device=dev)
    with pytest.raises(duo.DuoError) as e:
        duo.mixed_forward(q, kv, kv, a, softmax_scale=0.125, lambda_block=32)
    assert e.value.status == 2
