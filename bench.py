"""Benchmark of the DuoAttention hot path on one MI355X.

Default: the Llama-2-7B decode layer (MHA 32 heads x 128, bf16, 32768-token
context, 8 retrieval heads, 24 streaming heads with a 16 + 64 ring). A step is
one duo_decode call: the append of the new token to both caches, split-K
retrieval attention over the full cache, streaming attention over the ring and
the split merge -- one fused kernel launch.

The 134 MB retrieval cache of one layer fits in the 256 MB MALL, so the
timed loop cycles over `--layers` independent layers (8 x 134 MB by default),
as a model's decode step visits its layers; every step's KV bytes then come
from HBM. Inputs are synthetic (seeded N(0,1) drawn on the device) and
resident in HBM before the timed region. One JSON line is printed.

`--gpus N` with N > 1 is refused: this build measures one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, vendor figure


def _decode_step_bytes(n, Hr, Hs, Hq, Hkv, D, W, e=2):
    """Algorithmic bytes of one decode step at position n: every cached K/V
    byte read once, q read, out written, new K/V read and written once."""
    retrieval = Hr * (n + 1) * D * 2 * e
    streaming = Hs * min(n + 1, W) * D * 2 * e
    return retrieval + streaming + Hq * D * 2 * 2 + Hkv * D * e * 2 * 2


def bench_decode(args, dev):
    import torch
    import kv_cache_compression_duo_amd as duo
    from duo_synth import WORKLOADS, device_normal

    w = WORKLOADS["llama2_7b_decode_32k"]
    Hq, Hkv, D, Hr = w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_retrieval_kv
    Hs = Hkv - Hr
    ctx, L = w.context, args.layers
    total = args.warmup + args.steps
    per_layer = (total + L - 1) // L
    layers = []
    for li in range(L):
        lay = duo.DuoLayer(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, n_retrieval_kv_heads=Hr,
                           capacity=ctx + per_layer, softmax_scale=w.softmax_scale, device=dev)
        chunk = 4096
        for a in range(0, ctx, chunk):
            k = device_normal((1, chunk, Hkv, D), 7000 + li * 100 + a // chunk, dev, torch.bfloat16)
            v = device_normal((1, chunk, Hkv, D), 9000 + li * 100 + a // chunk, dev, torch.bfloat16)
            lay.append_kv(k, v)
        layers.append(lay)
    q = (device_normal((total, 1, 1, Hq, D), 11, dev, torch.float32) / math.sqrt(D)).to(torch.bfloat16)
    kn = device_normal((total, 1, 1, Hkv, D), 12, dev, torch.bfloat16)
    vn = device_normal((total, 1, 1, Hkv, D), 13, dev, torch.bfloat16)
    out = torch.empty((1, 1, Hq, D), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()
    for s in range(args.warmup):
        layers[s % L].decode(q[s], kn[s], vn[s], out)
    torch.cuda.synchronize()
    # timed region 1: the plain step loop (value, ms_per_step)
    steps_a = args.steps // 2
    steps_b = args.steps - steps_a
    nbytes_a = 0
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(steps_a):
        s = args.warmup + i
        lay = layers[s % L]
        nbytes_a += _decode_step_bytes(lay.n_tokens, Hr, Hs, Hq, Hkv, D, w.sink + w.recent)
        lay.decode(q[s], kn[s], vn[s], out)
    t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    # timed region 2: HIP events around every launch of the decode kernel on
    # the stream it runs on (average launch duration for the roofline)
    nbytes_b = 0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps_b)]
    for i in range(steps_b):
        s = args.warmup + steps_a + i
        lay = layers[s % L]
        nbytes_b += _decode_step_bytes(lay.n_tokens, Hr, Hs, Hq, Hkv, D, w.sink + w.recent)
        ev[i][0].record()
        lay.decode(q[s], kn[s], vn[s], out)
        ev[i][1].record()
    torch.cuda.synchronize()
    kern_ms = [a.elapsed_time(b) for a, b in ev]
    avg_kern_ms = sum(kern_ms) / len(kern_ms)
    ms_step = total_ms / steps_a
    gbs = nbytes_a / (total_ms * 1e-3) / 1e9
    achieved = (nbytes_b / steps_b) / (avg_kern_ms * 1e-3) / 1e9
    nbytes = nbytes_a
    res = {
        "value": gbs, "ms_per_step": ms_step, "tok_per_s": 1000.0 / ms_step,
        "bytes_per_step": nbytes / steps_a,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "decode_kernel<128,1,bf16>",
                     "avg_launch_us": avg_kern_ms * 1e3},
        "layers_cycled": L,
    }
    return res


def cpu_baseline_decode(budget_s: float):
    """The oracle's decode step timed on the host: the Llama-2-7B layer at a
    32768-token context, repeated until `budget_s` seconds have elapsed."""
    import numpy as np
    import oracle
    from duo_synth import WORKLOADS, make_inputs
    w = WORKLOADS["llama2_7b_decode_32k"]
    inp = make_inputs(w, steps=64)
    orc = oracle.OracleLayer(w.n_q_heads, w.n_kv_heads, w.head_dim, inp.retrieval_mask,
                             w.softmax_scale, w.sink, w.recent)
    orc.append(inp.k, inp.v)
    nbytes = 0
    t0 = time.perf_counter()
    steps = 0
    while steps < 64:
        n = orc.n
        orc.decode(inp.q_steps[steps], inp.k_steps[steps], inp.v_steps[steps])
        nbytes += _decode_step_bytes(n, w.n_retrieval_kv, w.n_kv_heads - w.n_retrieval_kv,
                                     w.n_q_heads, w.n_kv_heads, w.head_dim, w.sink + w.recent)
        steps += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = 1
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": f"{steps} oracle decode steps of the 32x128 layer at 32768 context "
                      f"({dt:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported in this build",
              file=sys.stderr)
        sys.exit(2)
    import torch
    dev = torch.device("cuda:0")
    r = bench_decode(args, dev)
    line = {
        "metric": "duo-attn decode KV GB/s & tok/s; chunked-prefill TFLOP/s, Llama-3-8B layer",
        "value": r["value"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": r["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama2_7b_decode_32k", "heads": "32x128 MHA, 8 retrieval",
                   "context": 32768, "layers_cycled": r["layers_cycled"]},
        "tok_per_s": r["tok_per_s"],
        "roofline": r["roofline"],
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
