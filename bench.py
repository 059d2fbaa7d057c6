"""Benchmark of the DuoAttention hot path on one MI355X.

Headline (the JSON line's `value`): the Llama-2-7B decode layer -- MHA 32
heads x 128, bf16, 32768-token context, 8 retrieval heads with the full cache,
24 streaming heads with a 16 + 64 ring. A step is one duo_decode call (append
of the new token to both caches, split-K retrieval attention, ring attention,
split merge: one fused kernel launch). `value` is algorithmic KV GB/s (every
cached K/V byte read once per step plus q/out/new-token traffic), `tok_per_s`
the decode steps per second of this layer.

The 134 MB retrieval cache of one layer fits in the 256 MB MALL, so the
timed loop cycles over `--layers` independent layers (8 x 134 MB), as a
model's decode step visits its layers; every step's KV bytes then come from
HBM. Inputs are synthetic (seeded N(0,1) drawn on the device) and resident in
HBM before any timed region.

The same line carries the other workloads under "workloads": the 8-head D=64
layer (prefill 1024 + 16 decode steps, latency), the Llama-3-8B GQA chunked
prefill (65536 tokens in 8192-token chunks, TFLOP/s), the alpha-blend mixed
forward (Llama-2-7B shape, 16384 tokens, TFLOP/s), its gradient with respect
to the gates at the same size (TFLOP/s over the same attention pairs) and the
Llama-3-8B 4-bit decode at a 1,048,576-token context (KV GB/s, tok/s).

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


# ---- algorithmic work ------------------------------------------------------------
def decode_step_bytes(n, Hr, Hs, Hq, Hkv, D, W, kv_bytes_per_token_head, ring_elem=2):
    """Bytes one decode step at position n must move: every cached K/V byte
    read once (retrieval rows 0..n, ring slots), q read, out written, the new
    token's K/V read once and written once to its cache."""
    retrieval = Hr * (n + 1) * kv_bytes_per_token_head
    streaming = Hs * min(n + 1, W) * D * 2 * ring_elem
    q_out = Hq * D * 2 * 2
    new_read = Hkv * D * 2 * ring_elem
    new_write = Hr * kv_bytes_per_token_head + Hs * D * 2 * ring_elem
    return retrieval + streaming + q_out + new_read + new_write


def causal_pairs(T0, T):
    """Allowed (query, key) pairs of T causal queries at positions T0..T0+T-1."""
    return T * T0 + T * (T + 1) // 2


def lambda_pairs(T0, T, S, R):
    """Allowed pairs under the Lambda mask (sink S, recent R incl. the query):
    query i sees i + 1 keys while i + 1 <= S + R, else S + R keys."""
    W = S + R
    tot = 0
    lo, hi = T0, T0 + T
    a, b = lo, min(hi, W)
    if b > a:
        tot += (b * (b + 1) - a * (a + 1)) // 2
    a = max(lo, W)
    if hi > a:
        tot += (hi - a) * W
    return tot


# ---- timing helpers --------------------------------------------------------------
def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def _lead(torch):
    """Queue about half a millisecond of device-side waiting ahead of a start
    event, so that the host has queued the timed launches before the event
    fires: a region of few launches then measures device time, not the
    host's launch latency for its first call."""
    if hasattr(torch.cuda, "_sleep"):
        torch.cuda._sleep(1_000_000)


def time_region(torch, fn, reps=1):
    a, b = _events(torch)
    torch.cuda.synchronize()
    _lead(torch)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


# ---- measured HBM traffic (rocprofv3 counters) -------------------------------------
# A decode kernel's HBM bytes per launch come from two rocprofv3 --pmc runs of
# `bench.py --traffic-probe` (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch),
# each scaled by what the same counter reads for a device copy of known size in
# the same run. `bench.py --traffic-summary FETCH_DIR WRITE_DIR` turns the two
# runs into one record per kernel under profiles/ (.json, read here, and .md).
# A figure is reported only while the kernel's sources hash to the value
# recorded with it.
TRAFFIC = {
    "decode": dict(
        kernel="decode_kernel<128, 1, duo::Bf16Tag>", workload="llama2_7b_decode_32k",
        json=os.path.join(ROOT, "profiles", "decode_kernel_llama2_7b_32k_traffic.json"),
        sources=["k_decode.hip", "decode_common.hpp", "decode_mma.hpp", "mfma_common.hpp",
                 "split_merge.hpp", "device_common.hpp", "duo_api.cpp", "duo_internal.hpp"]),
    "int4": dict(
        kernel="decode_int4_kernel<128, 4, duo::Fp16Tag>", workload="llama3_8b_int4_decode_1m",
        json=os.path.join(ROOT, "profiles", "decode_int4_kernel_llama3_8b_1m_traffic.json"),
        sources=["k_decode_int4.hip", "int4_codec.hpp", "decode_common.hpp", "split_merge.hpp",
                 "device_common.hpp", "duo_api.cpp", "duo_internal.hpp"]),
}
COPY_BYTES = 256 << 20


def source_hash(key: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC[key]["sources"]:
        with open(os.path.join(ROOT, "kv_cache_compression_duo_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def measured_traffic(key: str = "decode"):
    try:
        with open(TRAFFIC[key]["json"]) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash(key):
        return None  # the kernel changed since the counters were taken
    return t.get("bytes_per_launch")


def traffic_probe(dev):
    """Launches profiled by the two counter runs: decode steps of one layer of
    the Llama-2 workload, decode steps of the 1M-token 4-bit layer, then a
    plain device copy of COPY_BYTES."""
    import torch
    import kv_cache_compression_duo_amd as duo
    from duo_synth import WORKLOADS, device_normal

    w = WORKLOADS["llama2_7b_decode_32k"]
    Hq, Hkv, D, Hr = w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_retrieval_kv
    steps = 6
    lay = duo.DuoLayer(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, n_retrieval_kv_heads=Hr,
                       capacity=w.context + steps, softmax_scale=w.softmax_scale, device=dev)
    for a in range(0, w.context, 8192):
        lay.append_kv(device_normal((1, 8192, Hkv, D), 7000 + a // 8192, dev, torch.bfloat16),
                      device_normal((1, 8192, Hkv, D), 9000 + a // 8192, dev, torch.bfloat16))
    q = (device_normal((steps, 1, 1, Hq, D), 11, dev, torch.float32) / math.sqrt(D)).to(torch.bfloat16)
    kn = device_normal((steps, 1, 1, Hkv, D), 12, dev, torch.bfloat16)
    vn = device_normal((steps, 1, 1, Hkv, D), 13, dev, torch.bfloat16)
    out = torch.empty((1, 1, Hq, D), dtype=torch.bfloat16, device=dev)
    for s in range(steps):
        lay.decode(q[s], kn[s], vn[s], out)
    del lay
    w4 = WORKLOADS["llama3_8b_int4_decode_1m"]
    Hq, Hkv, D, Hr = w4.n_q_heads, w4.n_kv_heads, w4.head_dim, w4.n_retrieval_kv
    steps4 = 4
    lay4 = duo.DuoLayer(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, n_retrieval_kv_heads=Hr,
                        capacity=w4.context + steps4, softmax_scale=w4.softmax_scale,
                        kv_dtype="fp16", retrieval_dtype="int4", device=dev)
    for a in range(0, w4.context, 65536):
        lay4.append_kv(device_normal((1, 65536, Hkv, D), 5000 + a // 65536, dev, torch.float16),
                       device_normal((1, 65536, Hkv, D), 6000 + a // 65536, dev, torch.float16))
    q4 = device_normal((steps4, 1, 1, Hq, D), 51, dev, torch.bfloat16)
    kn4 = device_normal((steps4, 1, 1, Hkv, D), 52, dev, torch.float16)
    vn4 = device_normal((steps4, 1, 1, Hkv, D), 53, dev, torch.float16)
    out4 = torch.empty((1, 1, Hq, D), dtype=torch.bfloat16, device=dev)
    for s in range(steps4):
        lay4.decode(q4[s], kn4[s], vn4[s], out4)
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"# traffic probe: {steps} + {steps4} decode launches, 3 copies of {COPY_BYTES} bytes",
          file=sys.stderr, flush=True)


def _csv_rows(run_dir, suffix):
    import csv
    import glob
    for f in sorted(glob.glob(os.path.join(run_dir, "**", "*" + suffix), recursive=True)):
        with open(f, newline="") as fh:
            yield from csv.DictReader(fh)


def _pmc_values(run_dir, counter):
    """Counter values per dispatch, by kernel name, from a rocprofv3 csv run."""
    vals = {}
    for row in _csv_rows(run_dir, "counter_collection.csv"):
        if row.get("Counter_Name") == counter:
            vals.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    return vals


def _pmc_means(run_dir, counter):
    return {k: sum(v) / len(v) for k, v in _pmc_values(run_dir, counter).items()}


def traffic_summary(fetch_dir, write_dir):
    fetch = _pmc_means(fetch_dir, "FETCH_SIZE")
    write = _pmc_means(write_dir, "WRITE_SIZE")

    def pick(d, key):
        names = [k for k in d if key in k]
        if len(names) != 1:
            raise SystemExit(f"expected one kernel matching {key!r}, found {names}")
        return names[0], d[names[0]]
    copy_name, f_copy = pick(fetch, "__amd_rocclr_copyBuffer")
    _, w_copy = pick(write, "__amd_rocclr_copyBuffer")
    kib = COPY_BYTES / 1024.0
    f_scale, w_scale = kib / f_copy, kib / w_copy
    for key, spec in TRAFFIC.items():
        name, f_k = pick(fetch, spec["kernel"])
        _, w_k = pick(write, spec["kernel"])
        fetch_b = f_k * f_scale * 1024.0
        write_b = w_k * w_scale * 1024.0
        t = {"kernel": name, "workload": spec["workload"],
             "fetch_kib_per_launch": f_k, "write_kib_per_launch": w_k,
             "copy_kernel": copy_name, "copy_bytes": COPY_BYTES,
             "copy_fetch_kib": f_copy, "copy_write_kib": w_copy,
             "fetch_scale": f_scale, "write_scale": w_scale,
             "fetch_bytes_per_launch": fetch_b, "write_bytes_per_launch": write_b,
             "bytes_per_launch": fetch_b + write_b, "source_hash": source_hash(key)}
        os.makedirs(os.path.dirname(spec["json"]), exist_ok=True)
        with open(spec["json"], "w") as fh:
            json.dump(t, fh, indent=1)
        print(json.dumps(t, indent=1))


def kernel_summary(trace_dir, group=8):
    """Markdown table of the library's kernels in a rocprofv3 --kernel-trace
    csv run: calls and durations, and for the flash kernels the totals of
    consecutive groups of `group` dispatches (one per prefill pass of 8
    chunks), in dispatch order."""
    per = {}
    for row in _csv_rows(trace_dir, "kernel_trace.csv"):
        name = row["Kernel_Name"]
        if "duo::" not in name:
            continue
        t0, t1 = int(row["Start_Timestamp"]), int(row["End_Timestamp"])
        per.setdefault(name, []).append((t0, (t1 - t0) / 1000.0))
    print("| kernel | calls | average us | min us | max us | total ms |")
    print("|---|---:|---:|---:|---:|---:|")
    for name, v in sorted(per.items(), key=lambda kv: -sum(d for _, d in kv[1])):
        d = [x for _, x in sorted(v)]
        print(f"| `{name}` | {len(d)} | {sum(d) / len(d):.2f} | {min(d):.2f} | {max(d):.2f} "
              f"| {sum(d) / 1000:.3f} |")
    print()
    for name, v in sorted(per.items()):
        if "attn_kernel<128, 4, 0>" not in name and "attn_kernel<128, 4, 1>" not in name:
            continue
        d = [x for _, x in sorted(v)]
        passes = [sum(d[i:i + group]) / 1000 for i in range(0, len(d) - group + 1, group)]
        print(f"`{name}`: totals of successive groups of {group} dispatches (ms): "
              + ", ".join(f"{x:.3f}" for x in passes))
    # the headline decode runs twice per bench: its steps cycling over several
    # layers, then the same number of steps on one layer (warm); each leg
    # starts with `group` warm-up steps
    for name, v in sorted(per.items()):
        if "decode_kernel<128, 1," not in name:
            continue
        d = [x for _, x in sorted(v)]
        h = len(d) // 2
        legs = [d[group:h], d[h + group:]]
        if all(legs):
            print(f"`{name}`: average of the timed dispatches of the cycled-layer leg "
                  f"{sum(legs[0]) / len(legs[0]):.2f} us ({len(legs[0])}), of the one-layer "
                  f"(warm) leg {sum(legs[1]) / len(legs[1]):.2f} us ({len(legs[1])})")


def counter_summary(*run_dirs):
    """Per-dispatch averages of every counter in rocprofv3 --pmc csv runs, by
    kernel, with the dispatch duration where the run records it."""
    rows = {}
    for rd in run_dirs:
        for row in _csv_rows(rd, "counter_collection.csv"):
            name = row["Kernel_Name"]
            if "duo::" not in name:
                continue
            rows.setdefault(name, {}).setdefault(row["Counter_Name"], []).append(
                float(row["Counter_Value"]))
            if row.get("Start_Timestamp") and row.get("End_Timestamp"):
                rows[name].setdefault("_duration_us@" + rd, []).append(
                    (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1000.0)
    out = {}
    for name, cs in rows.items():
        out[name] = {c: sum(v) / len(v) for c, v in cs.items()}
    print(json.dumps(out, indent=1))


# ---- workloads -------------------------------------------------------------------
def bench_decode_llama2(args, dev):
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
        chunk = 8192
        for a in range(0, ctx, chunk):
            k = device_normal((1, chunk, Hkv, D), 7000 + li * 100 + a // chunk, dev, torch.bfloat16)
            v = device_normal((1, chunk, Hkv, D), 9000 + li * 100 + a // chunk, dev, torch.bfloat16)
            lay.append_kv(k, v)
        layers.append(lay)
    q = (device_normal((total, 1, 1, Hq, D), 11, dev, torch.float32) / math.sqrt(D)).to(torch.bfloat16)
    kn = device_normal((total, 1, 1, Hkv, D), 12, dev, torch.bfloat16)
    vn = device_normal((total, 1, 1, Hkv, D), 13, dev, torch.bfloat16)
    out = torch.empty((1, 1, Hq, D), dtype=torch.bfloat16, device=dev)
    W = w.sink + w.recent
    torch.cuda.synchronize()
    for s in range(args.warmup):
        layers[s % L].decode(q[s], kn[s], vn[s], out)
    torch.cuda.synchronize()
    n_before = [lay.n_tokens for lay in layers]
    nbytes = 0
    for i in range(args.steps):
        li = (args.warmup + i) % L
        nbytes += decode_step_bytes(n_before[li] + i // L, Hr, Hs, Hq, Hkv, D, W, D * 2 * 2)
    t0, t1 = _events(torch)
    t0.record()
    for i in range(args.steps):
        s = args.warmup + i
        layers[s % L].decode(q[s], kn[s], vn[s], out)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    ms_step = ms / args.steps
    gbs = nbytes / (ms * 1e-3) / 1e9
    # a step is exactly one launch of the decode kernel on the caller's stream,
    # so the events above bracket `steps` back-to-back launches of it
    del layers
    warm = decode_warm_llama2(args, dev, w, q, kn, vn, out)
    return {
        "value": gbs, "ms_per_step": ms_step, "tok_per_s": 1000.0 / ms_step,
        "bytes_per_step": nbytes / args.steps, "layers_cycled": L, "warm": warm,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": measured_traffic("decode"),
                     "kernel": "duo::decode_kernel<128, 1, duo::Bf16Tag>",
                     "avg_launch_us": ms_step * 1e3},
    }


def decode_warm_llama2(args, dev, w, q, kn, vn, out):
    """Secondary decode figure: the same steps back to back on ONE layer, whose
    134 MB cache stays resident in the 256 MB Infinity Cache between steps (warm,
    launch gaps included). Not the headline: a model's decode step visits all of
    its layers, so the headline cycles over several layers' caches."""
    import torch
    import kv_cache_compression_duo_amd as duo
    from duo_synth import device_normal

    Hq, Hkv, D, Hr = w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_retrieval_kv
    Hs, ctx, W = Hkv - Hr, w.context, w.sink + w.recent
    total = args.warmup + args.steps
    lay = duo.DuoLayer(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, n_retrieval_kv_heads=Hr,
                       capacity=ctx + total, softmax_scale=w.softmax_scale, device=dev)
    chunk = 8192
    for a in range(0, ctx, chunk):
        lay.append_kv(device_normal((1, chunk, Hkv, D), 7000 + a // chunk, dev, torch.bfloat16),
                      device_normal((1, chunk, Hkv, D), 9000 + a // chunk, dev, torch.bfloat16))
    torch.cuda.synchronize()
    for s in range(args.warmup):
        lay.decode(q[s], kn[s], vn[s], out)
    torch.cuda.synchronize()
    n0 = lay.n_tokens
    nbytes = sum(decode_step_bytes(n0 + i, Hr, Hs, Hq, Hkv, D, W, D * 2 * 2)
                 for i in range(args.steps))
    t0, t1 = _events(torch)
    t0.record()
    for i in range(args.steps):
        s = args.warmup + i
        lay.decode(q[s], kn[s], vn[s], out)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms_per_step": ms / args.steps, "kv_gbs": gbs, "frac_of_hbm_peak": gbs / HBM_PEAK_GBS,
            "layers_cycled": 1, "note": "one layer back to back, cache resident in the MALL"}


def bench_decode_gqa(args, dev):
    """Opt-in (--only gqa): the 16-bit decode of a Llama-3-8B-shaped layer (32
    query / 8 KV heads, head_dim 128, 32768-token context, 8 layers cycled) with
    4 and with 8 retrieval KV heads -- four query heads per KV head, the
    matrix-core decode loop. Not a headline workload."""
    import torch
    import kv_cache_compression_duo_amd as duo
    from duo_synth import device_normal

    Hq, Hkv, D, ctx, L, S, R = 32, 8, 128, 32768, args.layers, 16, 64
    total = args.warmup + args.steps
    per_layer = (total + L - 1) // L
    res = {}
    for Hr in (4, 8):
        layers = []
        for li in range(L):
            lay = duo.DuoLayer(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, n_retrieval_kv_heads=Hr,
                               capacity=ctx + per_layer, softmax_scale=D ** -0.5, sink=S,
                               recent=R, device=dev)
            for a in range(0, ctx, 8192):
                lay.append_kv(device_normal((1, 8192, Hkv, D), 7000 + li * 100 + a // 8192, dev,
                                            torch.bfloat16),
                              device_normal((1, 8192, Hkv, D), 9000 + li * 100 + a // 8192, dev,
                                            torch.bfloat16))
            layers.append(lay)
        q = device_normal((total, 1, 1, Hq, D), 11, dev, torch.bfloat16)
        kn = device_normal((total, 1, 1, Hkv, D), 12, dev, torch.bfloat16)
        vn = device_normal((total, 1, 1, Hkv, D), 13, dev, torch.bfloat16)
        out = torch.empty((1, 1, Hq, D), dtype=torch.bfloat16, device=dev)
        for s in range(args.warmup):
            layers[s % L].decode(q[s], kn[s], vn[s], out)
        torch.cuda.synchronize()
        n_before = [lay.n_tokens for lay in layers]
        nbytes = sum(decode_step_bytes(n_before[(args.warmup + i) % L] + i // L, Hr, Hkv - Hr, Hq,
                                       Hkv, D, S + R, D * 2 * 2) for i in range(args.steps))
        t0, t1 = _events(torch)
        t0.record()
        for i in range(args.steps):
            s = args.warmup + i
            layers[s % L].decode(q[s], kn[s], vn[s], out)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1)
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[f"retrieval_kv_heads_{Hr}"] = {"us_per_step": ms / args.steps * 1e3,
                                           "bytes_per_step": nbytes / args.steps, "kv_gbs": gbs,
                                           "hbm_frac": gbs / HBM_PEAK_GBS}
        del layers
    res["kernel"] = "duo::decode_kernel<128, 4, duo::Bf16Tag>"
    return res


def bench_mha8(args, dev):
    import torch
    import kv_cache_compression_duo_amd as duo
    from duo_synth import WORKLOADS, device_normal
    w = WORKLOADS["mha8_d64_seq1024"]
    H, D, T, steps = 8, 64, 1024, 16
    q = device_normal((1, T, H, D), 21, dev, torch.bfloat16)
    k = device_normal((1, T, H, D), 22, dev, torch.bfloat16)
    v = device_normal((1, T, H, D), 23, dev, torch.bfloat16)
    qs = device_normal((steps, 1, 1, H, D), 24, dev, torch.bfloat16)
    ks = device_normal((steps, 1, 1, H, D), 25, dev, torch.bfloat16)
    vs = device_normal((steps, 1, 1, H, D), 26, dev, torch.bfloat16)
    out = torch.empty_like(q)
    o1 = torch.empty((1, 1, H, D), dtype=torch.bfloat16, device=dev)
    layers = [duo.DuoLayer(n_q_heads=H, n_kv_heads=H, head_dim=D, n_retrieval_kv_heads=2,
                           capacity=T + steps, softmax_scale=w.softmax_scale, device=dev)
              for _ in range(6)]

    def run(lay):
        lay.prefill_chunk(q, k, v, out)
        for s in range(steps):
            lay.decode(qs[s], ks[s], vs[s], o1)

    run(layers[0])
    times = sorted(time_region(torch, lambda lay=lay: run(lay)) for lay in layers[1:])
    flops = (2 * causal_pairs(0, T) + 6 * lambda_pairs(0, T, 16, 64)) * 4 * D
    return {"ms_prefill_1024_plus_16_decode": times[len(times) // 2],
            "prefill_gflop": flops / 1e9}


def bench_prefill_llama3(args, dev):
    import torch
    import kv_cache_compression_duo_amd as duo
    from duo_synth import WORKLOADS, device_normal
    w = WORKLOADS["llama3_8b_prefill_64k"]
    Hq, Hkv, D, Hr = w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_retrieval_kv
    T, C = w.prefill_tokens, w.chunk
    qc = [device_normal((1, C, Hq, D), 310 + i, dev, torch.bfloat16) for i in range(T // C)]
    kc = [device_normal((1, C, Hkv, D), 320 + i, dev, torch.bfloat16) for i in range(T // C)]
    vc = [device_normal((1, C, Hkv, D), 330 + i, dev, torch.bfloat16) for i in range(T // C)]
    oc = [torch.empty_like(x) for x in qc]

    def one_pass():
        lay = duo.DuoLayer(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, n_retrieval_kv_heads=Hr,
                           capacity=T, softmax_scale=w.softmax_scale, device=dev)
        torch.cuda.synchronize()
        a, b = _events(torch)
        a.record()
        for i in range(len(qc)):
            lay.prefill_chunk(qc[i], kc[i], vc[i], oc[i])
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    one_pass()
    times = sorted(one_pass() for _ in range(args.prefill_reps))
    ms = times[len(times) // 2]
    G = Hq // Hkv
    ret_flops = Hr * G * causal_pairs(0, T) * 4 * D
    str_flops = (Hkv - Hr) * G * lambda_pairs(0, T, w.sink, w.recent) * 4 * D

    # The retrieval heads alone: a layer holding only the 4 retrieval KV heads
    # (16 query heads) prefilled with the same 8 chunks, so each chunk is the
    # append of its K/V rows plus one launch of the retrieval flash kernel
    # (the appends are about 10 us of a chunk's milliseconds).
    def retrieval_pass():
        lay = duo.DuoLayer(n_q_heads=Hr * G, n_kv_heads=Hr, head_dim=D, n_retrieval_kv_heads=Hr,
                           capacity=T, softmax_scale=w.softmax_scale, device=dev)
        torch.cuda.synchronize()
        a, b = _events(torch)
        a.record()
        for i in range(len(qr)):
            lay.prefill_chunk(qr[i], kr[i], vr[i], orr[i])
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    qr = [x[:, :, :Hr * G].contiguous() for x in qc]
    kr = [x[:, :, :Hr].contiguous() for x in kc]
    vr = [x[:, :, :Hr].contiguous() for x in vc]
    orr = [torch.empty_like(x) for x in qr]
    retrieval_pass()
    rtimes = sorted(retrieval_pass() for _ in range(args.prefill_reps))
    rms = rtimes[len(rtimes) // 2]
    return {"ms_full_prefill_8x8192": ms,
            "tflops_total": (ret_flops + str_flops) / (ms * 1e-3) / 1e12,
            "retrieval_tflop": ret_flops / 1e12, "streaming_tflop": str_flops / 1e12,
            "mfma_frac_total": (ret_flops + str_flops) / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "retrieval_ms": rms, "retrieval_tflops": ret_flops / (rms * 1e-3) / 1e12,
            "retrieval_mfma_frac": ret_flops / (rms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "retrieval_kernel": "duo::attn_kernel<128, 4, 0> (+ 8 appends of 8192 rows)"}


def block_lambda_pairs(T, S, R, b):
    """Allowed pairs of T queries (positions 0..T-1) under the block-sparse
    Lambda mask: key j visible to query i when j <= i and (j // b <
    ceil(S / b) or i // b - j // b < ceil(R / b))."""
    sb, rb = -(-S // b), -(-R // b)
    tot = 0
    for qb in range(-(-T // b)):
        for i in range(qb * b, min(T, qb * b + b)):
            lo_local = max(0, (qb - rb + 1) * b)
            sink_hi = min(sb * b, i + 1)
            tot += sink_hi + max(0, i + 1 - max(lo_local, sink_hi))
    return tot


def bench_mixed(args, dev):
    import torch
    import kv_cache_compression_duo_amd as duo
    from duo_synth import WORKLOADS, device_normal
    w = WORKLOADS["llama2_7b_mixed_16k"]
    H, D, T = w.n_q_heads, w.head_dim, w.mixed_tokens
    q = device_normal((1, T, H, D), 41, dev, torch.bfloat16)
    k = device_normal((1, T, H, D), 42, dev, torch.bfloat16)
    v = device_normal((1, T, H, D), 43, dev, torch.bfloat16)
    g = torch.Generator(device=dev)
    g.manual_seed(44)
    alpha = torch.rand((H,), generator=g, device=dev, dtype=torch.float32)
    out = torch.empty_like(q)
    fn = lambda: duo.mixed_forward(q, k, v, alpha, softmax_scale=w.softmax_scale, out=out)
    fn()
    ms = sorted(time_region(torch, fn) for _ in range(5))[2]
    flops = H * (causal_pairs(0, T) + lambda_pairs(0, T, w.sink, w.recent)) * 4 * D
    # the block-sparse Lambda form used while training the gates (64-token blocks)
    fb = lambda: duo.mixed_forward(q, k, v, alpha, softmax_scale=w.softmax_scale, out=out,  # noqa: E731
                                   lambda_block=64)
    fb()
    ms_b = sorted(time_region(torch, fb) for _ in range(5))[2]
    flops_b = H * (causal_pairs(0, T) + block_lambda_pairs(T, w.sink, w.recent, 64)) * 4 * D
    return {"ms": ms, "tflops": flops / (ms * 1e-3) / 1e12, "tflop": flops / 1e12,
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
            "block_sparse_ms": ms_b, "block_sparse_tflops": flops_b / (ms_b * 1e-3) / 1e12}


def bench_mixed_alpha_grad(args, dev):
    """Gradient with respect to the gates at the identification size: the
    same two attentions as the gate-blended forward (recomputed; no stored
    activations), dotted with dout, plus the per-head reduction."""
    import torch
    import kv_cache_compression_duo_amd as duo
    from duo_synth import WORKLOADS, device_normal
    w = WORKLOADS["llama2_7b_mixed_16k"]
    H, D, T = w.n_q_heads, w.head_dim, w.mixed_tokens
    q = device_normal((1, T, H, D), 41, dev, torch.bfloat16)
    k = device_normal((1, T, H, D), 42, dev, torch.bfloat16)
    v = device_normal((1, T, H, D), 43, dev, torch.bfloat16)
    dout = device_normal((1, T, H, D), 45, dev, torch.bfloat16)
    g = torch.Generator(device=dev)
    g.manual_seed(44)
    alpha = torch.rand((H,), generator=g, device=dev, dtype=torch.float32)
    grad = torch.empty(H, dtype=torch.float32, device=dev)
    ws = torch.empty(1 << 20, dtype=torch.uint8, device=dev)  # 8 KiB needed
    fn = lambda: duo.mixed_alpha_grad(q, k, v, dout, alpha, softmax_scale=w.softmax_scale,  # noqa: E731
                                      l1_weight=0.05, grad=grad, workspace=ws)
    fn()
    ms = sorted(time_region(torch, fn) for _ in range(5))[2]
    flops = H * (causal_pairs(0, T) + lambda_pairs(0, T, w.sink, w.recent)) * 4 * D
    return {"ms": ms, "tflops": flops / (ms * 1e-3) / 1e12, "tflop": flops / 1e12,
            "mfma_frac": flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}


def bench_int4_decode(args, dev):
    import torch
    import kv_cache_compression_duo_amd as duo
    from duo_synth import WORKLOADS, device_normal
    w = WORKLOADS["llama3_8b_int4_decode_1m"]
    Hq, Hkv, D, Hr = w.n_q_heads, w.n_kv_heads, w.head_dim, w.n_retrieval_kv
    Hs = Hkv - Hr
    N, steps, warm = w.context, args.int4_steps, 4
    lay = duo.DuoLayer(n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D, n_retrieval_kv_heads=Hr,
                       capacity=N + steps + warm, softmax_scale=w.softmax_scale, kv_dtype="fp16",
                       retrieval_dtype="int4", device=dev)
    chunk = 65536
    for a in range(0, N, chunk):
        kk = device_normal((1, chunk, Hkv, D), 5000 + a // chunk, dev, torch.float16)
        vv = device_normal((1, chunk, Hkv, D), 6000 + a // chunk, dev, torch.float16)
        lay.append_kv(kk, vv)
    total = steps + warm
    q = device_normal((total, 1, 1, Hq, D), 51, dev, torch.bfloat16)
    kn = device_normal((total, 1, 1, Hkv, D), 52, dev, torch.float16)
    vn = device_normal((total, 1, 1, Hkv, D), 53, dev, torch.float16)
    out = torch.empty((1, 1, Hq, D), dtype=torch.bfloat16, device=dev)
    for s in range(warm):
        lay.decode(q[s], kn[s], vn[s], out)
    torch.cuda.synchronize()
    n0 = lay.n_tokens
    nbytes = sum(decode_step_bytes(n0 + i, Hr, Hs, Hq, Hkv, D, w.sink + w.recent, 160)
                 for i in range(steps))
    t0, t1 = _events(torch)
    _lead(torch)
    t0.record()
    for i in range(steps):
        lay.decode(q[warm + i], kn[warm + i], vn[warm + i], out)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms_per_step": ms / steps, "tok_per_s": 1000.0 * steps / ms, "kv_gbs": gbs,
            "bytes_per_step": nbytes / steps, "hbm_frac": gbs / HBM_PEAK_GBS,
            "traffic": measured_traffic("int4"),
            "kernel": "duo::decode_int4_kernel<128, 4, duo::Fp16Tag>"}


def cpu_model() -> str:
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline_decode(budget_s: float):
    """The oracle's decode step timed on the host: the Llama-2-7B layer at a
    32768-token context, for the workload's 256 steps or until `budget_s`
    seconds have elapsed (input drawing and the context fill are not timed)."""
    import oracle
    from duo_synth import WORKLOADS, make_inputs
    w = WORKLOADS["llama2_7b_decode_32k"]
    inp = make_inputs(w)
    orc = oracle.OracleLayer(w.n_q_heads, w.n_kv_heads, w.head_dim, inp.retrieval_mask,
                             w.softmax_scale, w.sink, w.recent)
    orc.append(inp.k, inp.v)
    # the first steps' row arrays grow past the context; warm that up untimed
    orc.decode(inp.q_steps[0], inp.k_steps[0], inp.v_steps[0])
    Hr = w.n_retrieval_kv
    nbytes = 0
    t0 = time.perf_counter()
    steps = 0
    while steps + 1 < w.decode_steps:
        n = orc.n
        s = steps + 1
        orc.decode(inp.q_steps[s], inp.k_steps[s], inp.v_steps[s])
        nbytes += decode_step_bytes(n, Hr, w.n_kv_heads - Hr, w.n_q_heads, w.n_kv_heads,
                                    w.head_dim, w.sink + w.recent, w.head_dim * 4)
        steps += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    return {"value": nbytes / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "steps": steps, "ms_per_step": dt / max(steps, 1) * 1e3,
            "sample": f"{steps} oracle decode steps (steps 2..{steps + 1} of the workload's "
                      f"{w.decode_steps}) of the 32x128 layer at a 32768-token context, "
                      f"{dt:.1f} s; float64 NumPy, BLAS threads = cores; algorithmic bytes "
                      f"as for the GPU"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--int4-steps", type=int, default=64)
    ap.add_argument("--prefill-reps", type=int, default=3)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="",
                    help="comma list of: decode,mha8,prefill,mixed,grad,int4 (default: all), "
                         "and the opt-in gqa")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="run only the launches the counter runs measure")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 csv runs into the traffic records")
    ap.add_argument("--kernel-summary", metavar="TRACE_DIR",
                    help="markdown table of a rocprofv3 --kernel-trace csv run")
    ap.add_argument("--counter-summary", nargs="+", metavar="PMC_DIR",
                    help="per-kernel counter averages of rocprofv3 --pmc csv runs")
    args = ap.parse_args()
    if args.traffic_summary:
        traffic_summary(*args.traffic_summary)
        return
    if args.kernel_summary:
        kernel_summary(args.kernel_summary)
        return
    if args.counter_summary:
        counter_summary(*args.counter_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported in this build",
              file=sys.stderr)
        sys.exit(2)
    import torch
    dev = torch.device("cuda:0")
    if args.traffic_probe:
        traffic_probe(dev)
        return
    only = set(x for x in args.only.split(",") if x)
    want = lambda name: not only or name in only
    line = {
        "metric": "duo-attn decode KV GB/s & tok/s; chunked-prefill TFLOP/s, Llama-3-8B layer",
        "value": None, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "llama2_7b_decode_32k", "heads": "32x128 MHA, 8 retrieval",
                   "context": 32768, "layers_cycled": args.layers},
    }
    work = {}
    if want("decode"):
        r = bench_decode_llama2(args, dev)
        line["value"] = r["value"]
        line["ms_per_step"] = r["ms_per_step"]
        line["tok_per_s"] = r["tok_per_s"]
        line["roofline"] = r["roofline"]
        line["decode_warm"] = r["warm"]
        print(f"# decode llama2 32k: {r['value']:.0f} GB/s, {r['ms_per_step']*1e3:.1f} us/step",
              file=sys.stderr, flush=True)
    for name, key, fn in (("mha8", "mha8_d64_seq1024", bench_mha8),
                          ("prefill", "llama3_8b_prefill_64k", bench_prefill_llama3),
                          ("mixed", "llama2_7b_mixed_16k", bench_mixed),
                          ("grad", "llama2_7b_mixed_alpha_grad_16k", bench_mixed_alpha_grad),
                          ("int4", "llama3_8b_int4_decode_1m", bench_int4_decode)):
        if want(name):
            work[key] = fn(args, dev)
            print(f"# {key}: {json.dumps(work[key])}", file=sys.stderr, flush=True)
    if "gqa" in only:
        work["llama3_8b_decode_32k_gqa"] = bench_decode_gqa(args, dev)
        print(f"# llama3_8b_decode_32k_gqa: {json.dumps(work['llama3_8b_decode_32k_gqa'])}",
              file=sys.stderr, flush=True)
    line["workloads"] = work
    if want("decode") and not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_decode(args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
