"""GPU parity of the 4-bit retrieval cache: quantise-on-append codes against
the oracle bit for bit, and int4 decode against the oracle (which attends over
its own fma-dequantised cache) -- at a ragged context, across group sizes and
head dims, and at the full 1,048,576-token context of the Llama-3-8B layer."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from duo_synth import WORKLOADS, ContextStream, LayerInputs, make_inputs, rng, normal, round_fp16
from gpu_util import Routed, assert_blocks_close, assert_close, device, say, to_dev

pytestmark = pytest.mark.gpu

W5 = WORKLOADS["llama3_8b_int4_decode_1m"]


def _int4_layer(Hq, Hkv, D, nr, capacity, scale, kv_dtype="fp16", S=16, R=64):
    import kv_cache_compression_duo_amd as duo
    return duo.DuoLayer(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, n_retrieval_kv_heads=nr,
                        capacity=capacity, softmax_scale=scale, sink=S, recent=R,
                        kv_dtype=kv_dtype, retrieval_dtype="int4", device=device())


def _v_codes_per_token(vblocks, n, D):
    """[nblk, 16*D] block layout -> [n, D] codes. Channel ch, token m (low
    nibble) and m+16 (high nibble) of a block sit at byte
    16*(4*(16*(ch//64) + ch%16) + m//4) + 4*((ch%64)//16) + m%4."""
    vb = vblocks.cpu().numpy()
    p = np.arange(n)[:, None]
    ch = np.arange(D)[None, :]
    blk, m, hi = p // 32, (p % 32) % 16, (p % 32) >= 16
    off = 16 * (4 * (16 * (ch // 64) + ch % 16) + m // 4) + 4 * ((ch % 64) // 16) + m % 4
    byte = vb[blk, off]                        # [n, D]
    return np.where(hi, byte >> 4, byte & 0xF).astype(np.uint8)


def _sz_per_token(blocks, n):
    """[nblk, D/32, 32, 2] blocked scale/zero -> [n, D/32, 2]."""
    x = blocks.cpu().numpy().transpose(0, 2, 1, 3)  # [nblk, 32, D/32, 2]
    return x.reshape(-1, x.shape[2], 2)[:n]


@pytest.mark.parametrize("kv_dtype,D", [("fp16", 128), ("bf16", 128), ("fp16", 64)])
def test_int4_append_codes_bit_exact(kv_dtype, D):
    Hq, Hkv = 8, 2
    # single-token appends in the upper half of a 32-token block (after the
    # lower half was written) must leave the other tokens' nibbles alone
    pieces = [20, 1, 1, 30, 1, 1, 100, 5, 64, 1, 31, 1]
    n = sum(pieces)
    g = rng(500)
    k = normal(g, (n, Hkv, D)) * 2.0
    v = normal(g, (n, Hkv, D))
    rnd = round_fp16 if kv_dtype == "fp16" else (lambda x: torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    k, v = rnd(k), rnd(v)
    tdt = torch.float16 if kv_dtype == "fp16" else torch.bfloat16
    lay = _int4_layer(Hq, Hkv, D, 1, n + 3, 0.088, kv_dtype=kv_dtype)
    a = 0
    for c in pieces:
        lay.append_kv(to_dev(k[a:a + c], tdt)[None], to_dev(v[a:a + c], tdt)[None])
        a += c
    torch.cuda.synchronize()
    K, V, KS, VS = lay.retrieval_int4()
    ck, sk, zk = oracle.quantize_int4_g32(k[:, 0])
    cv, sv, zv = oracle.quantize_int4_g32(v[:, 0])
    got_k = K[0, 0, :n].cpu().numpy()
    np.testing.assert_array_equal(got_k, oracle.pack_nibbles(ck))
    np.testing.assert_array_equal(_v_codes_per_token(V[0, 0], n, D), cv)
    ks = _sz_per_token(KS[0, 0], n)
    vs = _sz_per_token(VS[0, 0], n)
    np.testing.assert_array_equal(ks[..., 0].view(np.uint16), sk.view(np.uint16))
    np.testing.assert_array_equal(ks[..., 1].view(np.uint16), zk.view(np.uint16))
    np.testing.assert_array_equal(vs[..., 0].view(np.uint16), sv.view(np.uint16))
    np.testing.assert_array_equal(vs[..., 1].view(np.uint16), zv.view(np.uint16))
    say(f"  {kv_dtype} D={D}: {n} tokens of K/V codes, scales and zero-points bit-exact")


@pytest.mark.parametrize("kv_dtype,D", [("fp16", 128), ("bf16", 128), ("fp16", 64)])
def test_int4_decode_writes_codes_bit_exact(kv_dtype, D):
    # the decode step quantises its new token into the 4-bit cache itself:
    # after steps that cross both nibble halves and a 32-token block boundary
    # every row's codes, scales and zero-points equal the oracle's
    Hq, Hkv, ctx, steps = 8, 2, 45, 40
    say(f"case: {kv_dtype} D={D}, context {ctx} then {steps} decode steps, codes checked")
    g = rng(510 + D)
    n = ctx + steps
    k = normal(g, (n, Hkv, D)) * 2.0
    v = normal(g, (n, Hkv, D))
    q = normal(g, (steps, Hq, D))
    rnd = round_fp16 if kv_dtype == "fp16" else (lambda x: torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    k, v = rnd(k), rnd(v)
    tdt = torch.float16 if kv_dtype == "fp16" else torch.bfloat16
    lay = _int4_layer(Hq, Hkv, D, 1, n, D ** -0.5, kv_dtype=kv_dtype)
    lay.append_kv(to_dev(k[:ctx], tdt)[None], to_dev(v[:ctx], tdt)[None])
    for s in range(steps):
        p = ctx + s
        lay.decode(to_dev(q[s])[None, None], to_dev(k[p], tdt)[None, None],
                   to_dev(v[p], tdt)[None, None])
    torch.cuda.synchronize()
    assert lay.n_tokens == n
    K, V, KS, VS = lay.retrieval_int4()
    ck, sk, zk = oracle.quantize_int4_g32(k[:, 0])
    cv, sv, zv = oracle.quantize_int4_g32(v[:, 0])
    np.testing.assert_array_equal(K[0, 0, :n].cpu().numpy(), oracle.pack_nibbles(ck))
    np.testing.assert_array_equal(_v_codes_per_token(V[0, 0], n, D), cv)
    ks = _sz_per_token(KS[0, 0], n)
    vs = _sz_per_token(VS[0, 0], n)
    np.testing.assert_array_equal(ks[..., 0].view(np.uint16), sk.view(np.uint16))
    np.testing.assert_array_equal(ks[..., 1].view(np.uint16), zk.view(np.uint16))
    np.testing.assert_array_equal(vs[..., 0].view(np.uint16), sv.view(np.uint16))
    np.testing.assert_array_equal(vs[..., 1].view(np.uint16), zv.view(np.uint16))
    say(f"  {n} rows of codes, scales and zero-points bit-exact after {steps} decode steps")


def _run_int4_decode(inp, context, steps, *, kv_dtype="fp16", label=""):
    w = inp.workload
    Hq, Hkv, D = inp.q_steps.shape[1], w.n_kv_heads, w.head_dim
    G = Hq // Hkv
    r = Routed(inp.retrieval_mask, G)
    tdt = torch.float16 if kv_dtype == "fp16" else torch.bfloat16
    lay = _int4_layer(Hq, Hkv, D, r.nr, context + steps, w.softmax_scale, kv_dtype, w.sink, w.recent)
    orc = oracle.OracleLayer(Hq, Hkv, D, inp.retrieval_mask, w.softmax_scale, w.sink, w.recent,
                             int4=True)
    if context:
        lay.append_kv(r.kv(to_dev(inp.k[:context], tdt))[None], r.kv(to_dev(inp.v[:context], tdt))[None])
        orc.append(inp.k[:context], inp.v[:context])
    rq = np.array([inp.retrieval_mask[h // G] for h in range(Hq)], bool)
    for s in range(steps):
        out = lay.decode(r.q(to_dev(inp.q_steps[s]))[None, None],
                         r.kv(to_dev(inp.k_steps[s], tdt))[None, None],
                         r.kv(to_dev(inp.v_steps[s], tdt))[None, None])
        ref = orc.decode(inp.q_steps[s], inp.k_steps[s], inp.v_steps[s])
        assert_blocks_close(r.out(out)[0, 0].float().cpu().numpy(), ref, rq,
                            f"{label} step {s}", head_axis=0)
    assert lay.n_tokens == context + steps


def test_int4_decode_llama3_ragged():
    say(f"case: {W5.key} context 3001 + 4 decode")
    inp = make_inputs(W5, tokens=3001, steps=4)
    _run_int4_decode(inp, 3001, 4, label=W5.key)


@pytest.mark.parametrize("context", [0, 1, 31, 32, 33, 700])
def test_int4_decode_contexts(context):
    w = dataclasses.replace(W5, n_q_heads=8, n_kv_heads=2, fixed_retrieval=(1,))
    say(f"case: int4 decode context={context}")
    inp = make_inputs(w, tokens=max(context, 1), steps=3, seed=5100 + context)
    _run_int4_decode(inp, context, 3, label=f"ctx{context}")


@pytest.mark.parametrize("G,D,ring", [(1, 128, "fp16"), (2, 128, "fp16"), (1, 64, "bf16"),
                                      (8, 64, "fp16"), (4, 128, "bf16")])
def test_int4_decode_shapes(G, D, ring):
    w = dataclasses.replace(W5, n_q_heads=2 * G, n_kv_heads=2, head_dim=D, fixed_retrieval=(0,),
                            softmax_scale=D ** -0.5, ring_dtype=ring)
    say(f"case: int4 decode G={G} D={D} ring={ring}")
    inp = make_inputs(w, tokens=450, steps=3, seed=5200 + G + D)
    _run_int4_decode(inp, 450, 3, kv_dtype=ring, label=f"G{G}D{D}{ring}")


def test_int4_rejects_too_many_columns():
    import kv_cache_compression_duo_amd as duo
    with pytest.raises(duo.DuoError) as e:
        _int4_layer(16, 2, 128, 1, 64, 0.088)  # G = 8 with D = 128
    assert e.value.status == 2


def test_int4_decode_full_context_1m():
    """The 1,048,576-token layer: context streamed to the GPU in 64K chunks,
    two decode steps checked for the first and last retrieval KV head (8
    query heads) and every streaming head."""
    w = W5
    cs = ContextStream(w, steps=2)
    ks, vs = [], []
    for k, v in cs.chunks():
        ks.append(k.astype(np.float16))
        vs.append(v.astype(np.float16))
    inp = cs.tail(LayerInputs(workload=w, retrieval_mask=np.zeros(w.n_kv_heads, np.uint8)))
    N = w.context
    G = w.n_q_heads // w.n_kv_heads
    r = Routed(inp.retrieval_mask, G)
    say(f"case: {w.key} context {N}, retrieval KV heads {r.perm[:r.nr]}")
    lay = _int4_layer(w.n_q_heads, w.n_kv_heads, w.head_dim, r.nr, N + 2, w.softmax_scale,
                      "fp16", w.sink, w.recent)
    for k, v in zip(ks, vs):
        lay.append_kv(r.kv(torch.from_numpy(k).cuda())[None], r.kv(torch.from_numpy(v).cuda())[None])
    torch.cuda.synchronize()
    ret_heads = [h for h in range(w.n_kv_heads) if inp.retrieval_mask[h]]
    str_heads = [h for h in range(w.n_kv_heads) if not inp.retrieval_mask[h]]
    check_ret = [ret_heads[0], ret_heads[-1]]
    deq = {}
    for h in check_ret:
        kk = np.concatenate([x[:, h] for x in ks]).astype(np.float32)
        vv = np.concatenate([x[:, h] for x in vs]).astype(np.float32)
        deq[h] = [oracle.dequantize_int4_g32(*oracle.quantize_int4_g32(kk)),
                  oracle.dequantize_int4_g32(*oracle.quantize_int4_g32(vv))]
    keep = np.concatenate([np.arange(w.sink), np.arange(N - w.recent, N)])
    ring_k = {h: np.concatenate([x[:, h] for x in ks])[keep].astype(np.float64) for h in str_heads}
    ring_v = {h: np.concatenate([x[:, h] for x in vs])[keep].astype(np.float64) for h in str_heads}
    pos = list(keep)
    for s in range(2):
        n = N + s
        out = lay.decode(r.q(to_dev(inp.q_steps[s]))[None, None],
                         r.kv(to_dev(inp.k_steps[s], torch.float16))[None, None],
                         r.kv(to_dev(inp.v_steps[s], torch.float16))[None, None])
        got = r.out(out)[0, 0].float().cpu().numpy()
        for h in check_ret:
            kn = oracle.dequantize_int4_g32(*oracle.quantize_int4_g32(inp.k_steps[s][h][None]))
            vn = oracle.dequantize_int4_g32(*oracle.quantize_int4_g32(inp.v_steps[s][h][None]))
            deq[h][0] = np.concatenate([deq[h][0], kn])
            deq[h][1] = np.concatenate([deq[h][1], vn])
            qh = inp.q_steps[s][h * G:(h + 1) * G]
            ref = oracle.masked_attention(qh, deq[h][0], deq[h][1], [n] * G, np.arange(n + 1),
                                          w.softmax_scale, "full")
            assert_close(got[h * G:(h + 1) * G], ref, f"1M step {s} retrieval kv{h}")
        pos.append(n)
        for h in str_heads:
            ring_k[h] = np.concatenate([ring_k[h], inp.k_steps[s][h][None]])
            ring_v[h] = np.concatenate([ring_v[h], inp.v_steps[s][h][None]])
        ref_s = np.concatenate([
            oracle.masked_attention(inp.q_steps[s][h * G:(h + 1) * G], ring_k[h], ring_v[h],
                                    [n] * G, pos, w.softmax_scale, "streaming", w.sink, w.recent)
            for h in str_heads])
        got_s = np.concatenate([got[h * G:(h + 1) * G] for h in str_heads])
        assert_close(got_s, ref_s, f"1M step {s} streaming")
