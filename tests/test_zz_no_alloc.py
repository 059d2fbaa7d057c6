"""The allocation-free gate gradient (duo_mixed_alpha_grad_noalloc): partial
sums in the library's device array instead of a caller workspace. Through the
C ABI it must give the same gradient as duo_mixed_alpha_grad_block with a
workspace (the same kernels and the same fixed-order reduction, so bit for
bit), on consecutive calls that reuse the array, the second one smaller; and
it must refuse a launch needing more partial slots than the array holds
before any HIP call."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from duo_synth import normal, random_case, rng, round_bf16


def _lib():
    from kv_cache_compression_duo_amd import _lib
    return _lib


def test_noalloc_refuses_more_partials_than_the_array_holds():
    """Host-side check (no GPU): fake, aligned pointers never reach a kernel."""
    L = _lib()
    f = L.lib.duo_mixed_alpha_grad_noalloc
    P = 0x1000
    # G = 1: one partial per 256-token tile of each (sequence, KV head)
    d = L.make_desc(batch=64, n_q_heads=32, n_kv_heads=32, head_dim=128, n_retrieval_kv_heads=0,
                    softmax_scale=0.088)
    fits = L.DUO_GRAD_SCRATCH_PARTIALS // (64 * 32) * 256  # 32 tiles of 256 tokens
    assert L.lib.duo_mixed_alpha_grad_workspace(ctypes.byref(d), fits) == \
        4 * L.DUO_GRAD_SCRATCH_PARTIALS
    assert f(ctypes.byref(d), P, P, P, P, P, 0.05, fits + 1, 0, P, None) == L.DUO_ERR_CAPACITY
    # other validation as for the workspace form
    assert f(ctypes.byref(d), P, P, P, P, P, 0.05, 0, 0, P, None) == L.DUO_ERR_INVALID_ARG
    assert f(ctypes.byref(d), P, P, P, P, P, 0.05, 100, 32, P, None) == L.DUO_ERR_UNSUPPORTED
    assert f(ctypes.byref(d), P, P, P, 0x1008, P, 0.05, 100, 0, P, None) == L.DUO_ERR_LAYOUT
    assert f(ctypes.byref(d), P, P, P, P, P, 0.05, 100, 0, None, None) == L.DUO_ERR_INVALID_ARG


def _inputs(seed, B, T, Hq, Hkv, D):
    qs, ks, vs, ds = [], [], [], []
    for b in range(B):
        q, k, v = random_case(seed + 7 * b, T=T, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D)
        qs.append(q)
        ks.append(k)
        vs.append(v)
        ds.append(round_bf16(normal(rng(seed + 7 * b + 1), (T, Hq, D))))
    return [np.stack(x) for x in (qs, ks, vs, ds)]


@pytest.mark.gpu
def test_noalloc_matches_workspace_entry_on_consecutive_calls():
    import kv_cache_compression_duo_amd as duo
    from gpu_util import device, grad_tolerance, say
    dev = device()
    # second call smaller than the first: fewer partial slots of the same array
    cases = [(2, 1000, 32, 8, 128, 16, 64, 0), (1, 300, 8, 8, 64, 4, 8, 64)]
    for i, (B, T, Hq, Hkv, D, S, R, blk) in enumerate(cases):
        say(f"case: no-alloc gate gradient call {i}: B={B} T={T} Hq={Hq} Hkv={Hkv} D={D} "
            f"S={S} R={R} lambda_block={blk}")
        q, k, v, dout = _inputs(31000 + 100 * i, B, T, Hq, Hkv, D)
        alpha = np.linspace(-0.5, 1.0, Hkv).astype(np.float32)
        t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).to(dev)  # noqa: E731
        a = torch.from_numpy(alpha).to(dev)
        kw = dict(softmax_scale=D ** -0.5, sink=S, recent=R, l1_weight=0.05, lambda_block=blk)
        ref = duo.mixed_alpha_grad(t(q), t(k), t(v), t(dout), a, **kw)
        got = torch.full((Hkv,), float("nan"), dtype=torch.float32, device=dev)
        duo.mixed_alpha_grad_noalloc(t(q), t(k), t(v), t(dout), a, got, **kw)
        torch.cuda.synchronize()
        g, r = got.cpu().numpy(), ref.cpu().numpy()
        say(f"  max |noalloc - workspace| = {np.abs(g - r).max():.3e}")
        assert np.array_equal(g, r), (g, r)
        if i == 1:  # the smaller case also against the oracle, within the derived bound
            o = oracle.mixed_alpha_grad(q[0], k[0], v[0], dout[0], alpha, D ** -0.5, S, R,
                                        l1_weight=0.05, block=blk)
            tol = grad_tolerance(q[0], k[0], v[0], dout[0], D ** -0.5, S, R, block=blk)
            assert np.all(np.abs(g - o) <= tol), (g, o, tol)
