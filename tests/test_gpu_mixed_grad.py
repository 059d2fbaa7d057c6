"""GPU parity of the gradient with respect to the gates of the gate-blended
forward (duo_mixed_alpha_grad, through the C ABI).

The kernel's only approximation is rounding the softmax weights P to bf16 for
the PV product (relative error at most 2^-9 per weight, the row sums taken
over the same rounded values), everything else accumulating in fp32. To first
order a weight error e_tj moves the gradient by w_tj * e_tj * dout_t . (v_j -
o_t); the roundings are independent, so by Hoeffding's inequality the total
stays within 6 * 2^-9 * sqrt(sum (w_tj * dout_t . (v_j - o_t))^2) over both
attentions (probability of exceeding it below 1e-7). The tests compute that
bound from fp64 attention weights, add 1e-5 of the summed magnitude for fp32
accumulation, and compare with the oracle: several group sizes and head
dims, ragged lengths, no sinks, a window covering the sequence, a batch of
two distinct sequences, and the gates' L1 term (positive, zero and negative
gates). At the Llama-2-7B identification size (16384 tokens, 32 heads) the
oracle gives the gradient of two KV heads, composed from its full and
streaming attention over blocks of query rows, within the same bound; and
every head's gradient must equal the forward difference
sum(dout * (mixed(alpha=1) - mixed(alpha=0))) taken from the forward kernel,
which rounds P identically, so only the forward's bf16 output rounding (at
most 2^-9 relative, independent) separates the two.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from duo_synth import WORKLOADS, device_normal, normal, random_case, rng, round_bf16
from gpu_util import device, grad_tolerance, grad_tolerance_rows, say, to_dev

pytestmark = pytest.mark.gpu


def _case(seed, T, Hq, Hkv, D, alpha):
    q, k, v = random_case(seed, T=T, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D)
    dout = round_bf16(normal(rng(seed + 1), (T, Hq, D)))
    return q, k, v, dout, np.asarray(alpha, np.float32)


def _gpu_grad(qs, ks, vs, douts, alpha, scale, S, R, l1):
    import kv_cache_compression_duo_amd as duo
    st = lambda xs: torch.stack([to_dev(x) for x in xs]).contiguous()  # noqa: E731
    a = torch.from_numpy(alpha).to(device())
    g = duo.mixed_alpha_grad(st(qs), st(ks), st(vs), st(douts), a, softmax_scale=scale, sink=S,
                             recent=R, l1_weight=l1)
    return g.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("T,Hq,Hkv,D,S,R", [
    (333, 8, 4, 128, 16, 64),   # GQA G=2, ragged length
    (200, 8, 8, 64, 16, 64),    # MHA, D=64
    (129, 16, 2, 128, 4, 8),    # G=8
    (97, 4, 1, 64, 0, 5),       # G=4, no sink tokens
    (300, 4, 4, 128, 1, 1),     # window of one
    (50, 4, 4, 128, 16, 64),    # S + R >= T: streaming equals full
])
def test_alpha_grad_matches_oracle(T, Hq, Hkv, D, S, R):
    dev = device()
    assert dev is not None
    scale, l1 = D ** -0.5, 0.05
    alpha = np.linspace(-0.25, 1.0, Hkv)
    alpha[0] = 0.0  # sign(0) = 0
    q, k, v, dout, alpha = _case(16000 + T + 7 * Hq + D + S, T, Hq, Hkv, D, alpha)
    say(f"case: alpha grad T={T} Hq={Hq} Hkv={Hkv} D={D} S={S} R={R}")
    got = _gpu_grad([q], [k], [v], [dout], alpha, scale, S, R, l1)
    ref = oracle.mixed_alpha_grad(q, k, v, dout, alpha, scale, S, R, l1_weight=l1)
    tol = grad_tolerance(q, k, v, dout, scale, S, R)
    say(f"  max |got - ref| = {np.abs(got - ref).max():.3e}, min tolerance {tol.min():.3e}, "
        f"max |ref| = {np.abs(ref).max():.3e}")
    assert np.all(np.abs(got - ref) <= tol), (got, ref, tol)


def test_alpha_grad_batch_of_two():
    device()
    T, Hq, Hkv, D, S, R = 260, 8, 2, 128, 16, 64
    scale, l1 = D ** -0.5, 0.05
    alpha = np.array([0.7, 0.2], np.float32)
    cases = [_case(17000 + 31 * b, T, Hq, Hkv, D, alpha) for b in range(2)]
    say(f"case: alpha grad batch 2, T={T}, distinct sequences")
    got = _gpu_grad([c[0] for c in cases], [c[1] for c in cases], [c[2] for c in cases],
                    [c[3] for c in cases], alpha, scale, S, R, l1)
    ref = sum(oracle.mixed_alpha_grad(c[0], c[1], c[2], c[3], alpha, scale, S, R)
              for c in cases) + l1 * np.sign(alpha)
    tol = sum(grad_tolerance(c[0], c[1], c[2], c[3], scale, S, R) for c in cases)
    assert np.all(np.abs(got - ref) <= tol), (got, ref, tol)


def test_alpha_grad_is_reproducible():
    device()
    T, Hq, Hkv, D = 700, 8, 4, 128
    alpha = np.full(Hkv, 0.5, np.float32)
    q, k, v, dout, alpha = _case(18000, T, Hq, Hkv, D, alpha)
    g1 = _gpu_grad([q], [k], [v], [dout], alpha, D ** -0.5, 16, 64, 0.0)
    g2 = _gpu_grad([q], [k], [v], [dout], alpha, D ** -0.5, 16, 64, 0.0)
    assert np.array_equal(g1, g2)


def test_alpha_grad_full_size_forward_difference():
    """The 16384-token MHA 32x128 identification layer (the bench's launch)."""
    import kv_cache_compression_duo_amd as duo
    dev = device()
    w = WORKLOADS["llama2_7b_mixed_16k"]
    T, H, D = w.mixed_tokens, w.n_q_heads, w.head_dim
    say(f"case: alpha grad full size T={T} H={H} D={D} against the forward difference")
    q = device_normal((1, T, H, D), 19001, dev, torch.bfloat16)
    k = device_normal((1, T, H, D), 19002, dev, torch.bfloat16)
    v = device_normal((1, T, H, D), 19003, dev, torch.bfloat16)
    dout = device_normal((1, T, H, D), 19004, dev, torch.bfloat16)
    alpha = torch.rand(H, generator=torch.Generator().manual_seed(19005)).to(dev)
    kw = dict(softmax_scale=w.softmax_scale, sink=w.sink, recent=w.recent)
    g = duo.mixed_alpha_grad(q, k, v, dout, alpha, l1_weight=0.05, **kw).double()
    o1 = duo.mixed_forward(q, k, v, torch.ones(H, device=dev), **kw).double()
    o0 = duo.mixed_forward(q, k, v, torch.zeros(H, device=dev), **kw).double()
    dd = dout.double()
    fd = (dd * (o1 - o0)).sum(dim=(0, 1, 3)) + 0.05 * torch.sign(alpha.double())
    bound = 6.0 * 2.0 ** -9 * torch.sqrt((dd ** 2 * (o1 ** 2 + o0 ** 2)).sum(dim=(0, 1, 3))) \
        + 1e-5 * (dd.abs() * (o1.abs() + o0.abs())).sum(dim=(0, 1, 3))
    err = (g - fd).abs()
    say(f"  max |grad - fd| = {err.max().item():.3e}, min bound {bound.min().item():.3e}, "
        f"max |fd| = {fd.abs().max().item():.3e}")
    assert torch.all(err <= bound), (g, fd, bound)


def test_alpha_grad_full_size_against_oracle():
    """The 16384-token MHA 32x128 identification layer, inputs drawn on the
    host: the gradient of KV heads 3 and 26 from the oracle, as the sum over
    the tokens and channels of dout * (full - streaming), each attention taken
    from oracle.masked_attention over blocks of 1024 query rows (a block's
    keys are the positions up to its last row; the masks remove the rest)."""
    import kv_cache_compression_duo_amd as duo
    dev = device()
    w = WORKLOADS["llama2_7b_mixed_16k"]
    T, H, D = w.mixed_tokens, w.n_q_heads, w.head_dim
    S, R, scale, l1 = w.sink, w.recent, w.softmax_scale, 0.05
    heads = (3, 26)
    say(f"case: alpha grad full size T={T} H={H} D={D}, heads {heads} against the oracle")
    g = rng(19100)
    q = round_bf16(normal(g, (T, H, D)))
    k = round_bf16(normal(g, (T, H, D)))
    v = round_bf16(normal(g, (T, H, D)))
    dout = round_bf16(normal(g, (T, H, D)))
    alpha = g.uniform(0.0, 1.0, size=H).astype(np.float32)
    got = _gpu_grad([q], [k], [v], [dout], alpha, scale, S, R, l1)
    pos = np.arange(T)
    ref = {}
    for h in heads:
        acc = 0.0
        for r0 in range(0, T, 1024):
            rows = pos[r0:r0 + 1024]
            hi = rows[-1] + 1
            full = oracle.masked_attention(q[rows, h], k[:hi, h], v[:hi, h], rows, pos[:hi],
                                           scale, "full")
            stream = oracle.masked_attention(q[rows, h], k[:hi, h], v[:hi, h], rows, pos[:hi],
                                             scale, "streaming", S, R)
            acc += float(np.sum(dout[rows, h].astype(np.float64) * (full - stream)))
        ref[h] = acc + l1 * float(np.sign(alpha[h]))
    tol = grad_tolerance_rows(q, k, v, dout, scale, S, R, heads)
    for h in heads:
        say(f"  head {h}: gpu {got[h]:.6f} oracle {ref[h]:.6f} |diff| "
            f"{abs(got[h] - ref[h]):.3e} bound {tol[h]:.3e}")
        assert abs(got[h] - ref[h]) <= tol[h], (h, got[h], ref[h], tol[h])
