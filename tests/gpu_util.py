"""Helpers for the GPU parity tests: device checks, head routing through the
C ABI, and the comparison at the tolerance the parity bar states
(max |o_gpu - o_ref| <= 2e-2 and ||o_gpu - o_ref|| / ||o_ref|| <= 5e-3,
in float64, separately over the retrieval and the streaming heads)."""
import sys

import numpy as np
import torch

MAX_ABS = 2e-2
REL_L2 = 5e-3


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU")
    import kv_cache_compression_duo_amd as duo  # fails loudly without libduo.so
    return torch.device("cuda:0")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype=torch.bfloat16, dev="cuda:0"):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(dtype).to(dev)


def errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.isfinite(got).all(), "non-finite GPU output"
    d = got - ref
    max_abs = float(np.abs(d).max()) if d.size else 0.0
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)) if d.size else 0.0
    return max_abs, rel


def assert_close(got, ref, label, max_abs=MAX_ABS, rel_l2=REL_L2):
    ma, rl = errors(got, ref)
    say(f"  {label}: max_abs={ma:.3e} rel_l2={rl:.3e}")
    assert ma <= max_abs and rl <= rel_l2, f"{label}: max_abs={ma:.3e} rel_l2={rl:.3e}"


def assert_blocks_close(got, ref, retrieval_q_heads, label, head_axis=-2):
    """Compare the retrieval-head and streaming-head blocks separately.
    ``retrieval_q_heads`` is a boolean per query head (original order)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    rmask = np.asarray(retrieval_q_heads, bool)
    if rmask.any():
        assert_close(np.take(got, np.where(rmask)[0], axis=head_axis),
                     np.take(ref, np.where(rmask)[0], axis=head_axis), label + " retrieval")
    if (~rmask).any():
        assert_close(np.take(got, np.where(~rmask)[0], axis=head_axis),
                     np.take(ref, np.where(~rmask)[0], axis=head_axis), label + " streaming")


class Routed:
    """Reorder heads with the library's permutation (retrieval first) on the way
    in and restore the caller's order on the way out."""

    def __init__(self, mask, G):
        from kv_cache_compression_duo_amd import head_permutation
        self.perm, self.nr = head_permutation(list(mask))
        self.G = G
        self.q_idx = torch.tensor([p * G + g for p in self.perm for g in range(G)])
        inv = [0] * len(self.q_idx)
        for i, p in enumerate(self.q_idx.tolist()):
            inv[p] = i
        self.q_inv = torch.tensor(inv)
        self.kv_idx = torch.tensor(self.perm)

    def q(self, t):   # [..., Hq, D] along dim -2
        return t.index_select(-2, self.q_idx.to(t.device)).contiguous()

    def kv(self, t):
        return t.index_select(-2, self.kv_idx.to(t.device)).contiguous()

    def out(self, t):
        return t.index_select(-2, self.q_inv.to(t.device)).contiguous()


def grad_tolerance(q, k, v, dout, scale, S, R, block=0):
    """Per-KV-head bound on |g_gpu - g_ref| for the gate gradient from the
    bf16 rounding of the softmax weights (relative error <= 2^-9 per weight,
    row sums over the same rounded values). To first order a weight error
    e_tj moves the gradient by w_tj * e_tj * dout_t . (v_j - o_t); the
    roundings are independent, so by Hoeffding's inequality the total stays
    within 6 * 2^-9 * sqrt(sum (w_tj * dout_t . (v_j - o_t))^2) over both
    attentions (exceeded with probability below 1e-7); 1e-5 of
    sum |dout * o| is added for fp32 accumulation. ``block`` > 0 takes the
    streaming mask block-sparse (64-token blocks in the kernel).

    The kernel also rounds q * scale * log2(e) once to bf16 (relative error
    eps_td <= 2^-9 per element), one query for both attentions. To first order
    that moves the gradient by sum_td eps_td * a_td with
    a_td = scale * q_td * sum_j (w^full_tj dv^full_tj - w^lam_tj dv^lam_tj) k_jd,
    dv_tj = dout_t . (v_j - o_t); these terms join the same Hoeffding sum."""
    q, k, v, dout = (np.asarray(x, np.float64) for x in (q, k, v, dout))
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    pos = np.arange(T)
    i, j = pos[:, None], pos[None, :]
    causal = j <= i
    if block:
        sb, rb = -(-S // block), -(-R // block)
        lam = causal & ((j // block < sb) | (i // block - j // block < rb))
    else:
        lam = causal & ((j < S) | (i - j < R))
    var = np.zeros(Hkv)
    mass = np.zeros(Hkv)
    for h in range(Hq):
        kv = h // G
        s = scale * q[:, h] @ k[:, kv].T
        wdv = []
        for allowed in (causal, lam):
            z = np.where(allowed, s, -np.inf)
            z -= z.max(axis=1, keepdims=True)
            w = np.exp(z)
            w /= w.sum(axis=1, keepdims=True)
            o = w @ v[:, kv]
            dv = dout[:, h] @ v[:, kv].T - np.sum(dout[:, h] * o, axis=1, keepdims=True)
            var[kv] += np.sum((w * dv) ** 2)
            mass[kv] += np.sum(np.abs(dout[:, h] * o))
            wdv.append(w * dv)
        a = scale * q[:, h] * ((wdv[0] - wdv[1]) @ k[:, kv])
        var[kv] += np.sum(a ** 2)
    return 6.0 * 2.0 ** -9 * np.sqrt(var) + 1e-5 * mass


def grad_tolerance_rows(q, k, v, dout, scale, S, R, kv_heads, rows_per_block=1024):
    """grad_tolerance for the KV heads ``kv_heads`` only, over query rows in
    blocks (each block sees keys up to its last row), for sequences too long
    for one T x T matrix. Returns {kv head: bound}."""
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = {}
    for kv in kv_heads:
        var = mass = 0.0
        for h in range(kv * G, kv * G + G):
            for r0 in range(0, T, rows_per_block):
                r1 = min(T, r0 + rows_per_block)
                i = np.arange(r0, r1)[:, None]
                j = np.arange(r1)[None, :]
                kk = np.asarray(k[:r1, kv], np.float64)
                vv = np.asarray(v[:r1, kv], np.float64)
                dd = np.asarray(dout[r0:r1, h], np.float64)
                s = scale * np.asarray(q[r0:r1, h], np.float64) @ kk.T
                causal = j <= i
                wdv = []
                for allowed in (causal, causal & ((j < S) | (i - j < R))):
                    z = np.where(allowed, s, -np.inf)
                    z -= z.max(axis=1, keepdims=True)
                    w = np.exp(z)
                    w /= w.sum(axis=1, keepdims=True)
                    o = w @ vv
                    dv = dd @ vv.T - np.sum(dd * o, axis=1, keepdims=True)
                    var += float(np.sum((w * dv) ** 2))
                    mass += float(np.sum(np.abs(dd * o)))
                    wdv.append(w * dv)
                a = scale * np.asarray(q[r0:r1, h], np.float64) * ((wdv[0] - wdv[1]) @ kk)
                var += float(np.sum(a ** 2))
        out[kv] = 6.0 * 2.0 ** -9 * np.sqrt(var) + 1e-5 * mass
    return out
