#!/usr/bin/env python3
"""Benchmark of the four-stream Engram saved-state gate on one MI355X.

A step is one pass of the whole hot path: engram_gate_fwd then
engram_gate_bwd over N = 8192 tokens (4 streams x 5120, the backward's
maximum N), mask Bernoulli(0.9), grad_out N(0,1), synthetic seeded inputs
already resident in HBM.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--rotate R] [--no-large] [--no-configs] [--no-cpu]
  python bench.py --configs [--no-cpu]     # one line per workload configuration 0-4

Consecutive steps use R (default 4) independent sets of inputs and outputs,
so no step finds its data in the 256 MB cache from the previous one.

The step's inputs are those of the N = 8192 forward workload (configuration
1: mask 0.9, no edge rows), run through forward and backward at the
backward's maximum N, the size of configuration 4.

The step rate (value, ms_per_step) is K steps back to back with nothing else
on the stream.  Also reported: forward-only and backward-only rates at
N = 8192, from HIP events around each call in a second pass of the same K
steps (each recorded event holds the stream for a few microseconds between
calls, so the events stay out of the rate's pass); a `configs` object with
the GPU time, tokens/s and fraction of 8 TB/s of each of the five workload
configurations (0: forward N = 64; 1: forward N = 8192; 2: forward +
backward N = 4096; 3: forward N = 1,048,512 in one launch; 4: forward +
backward N = 8192, mask 0.3 with edge rows, 1000 launches); GateConv; and
the fp64 CPU oracle's rate on a bounded sample of the step's workload.
"""
from __future__ import annotations

import argparse
import hashlib
import glob
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Engram gate tokens/s + achieved HBM GB/s (% of peak), fwd and fwd+bwd"
PEAK_GBPS = 8000.0          # MI355X HBM3E
N_STEP = 8192
N_LARGE = 1_048_512
SEED = 0
P_MASK = 0.9
FWD_BYTES_PER_TOKEN = 133_185   # X + KV + mask read, out + saved written
FWD_BYTES_FIXED = 81_920        # weight
BWD_BYTES_PER_TOKEN = 225_344   # X, KV, saved, grad_out read; grad_x, grad_kv written
BWD_BYTES_FIXED = 163_840       # weight read, grad_weight written


# GateConv ("Engram Operators", TileOPs): M sequences of T tokens, width d
GC_M, GC_T, GC_D = 4, 4096, 5120


def gc_fwd_bytes(M, T, d):
    """H, k, v read, Y and vhat written (bf16); alpha and rrms_h/k/v written
    (fp32); rms_w_h, rms_w_v, conv_w read (fp32)."""
    return M * T * (10 * d + 16) + 6 * d * 4


def gc_bwd_bytes(M, T, d):
    """dY, H, k, v, vhat and the four fp32 scalars read, dH, dk, dv written;
    the 6d fp32 weights read and their gradients written."""
    return M * T * (16 * d + 16) + 2 * 6 * d * 4


def fwd_bytes(n):
    return FWD_BYTES_PER_TOKEN * n + FWD_BYTES_FIXED


def bwd_bytes(n):
    return BWD_BYTES_PER_TOKEN * n + BWD_BYTES_FIXED


KERNEL_SOURCES = {  # what decides each recorded kernel's traffic: its code and its launch
    "fwd": ("engram_device.h", "engram_fwd.hip", "engram_api.cpp"),
    "fwd_large": ("engram_device.h", "engram_fwd.hip", "engram_api.cpp"),
    "bwd": ("engram_device.h", "engram_bwd.hip", "engram_api.cpp"),
    "gc_fwd": ("engram_device.h", "engram_gateconv.hip", "engram_api.cpp"),
    "gc_bwd": ("engram_device.h", "engram_gateconv.hip", "engram_api.cpp"),
}


def code_only(src):
    """C++ source without its comments, runs of whitespace collapsed: a comment
    edit leaves it (and the recorded traffic keyed on it) unchanged, a code
    edit does not.  String and character literals are kept whole."""
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
            out.append(" ")
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "memory_bound_engram_amd", "csrc", name), encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def recorded_traffic(kernel):
    """HBM bytes per launch from the rocprofv3 FETCH_SIZE/WRITE_SIZE runs, if
    they were taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    e = rec.get(kernel)
    if not e or e.get("source_hash") != kernel_source_hash(kernel):
        return None
    return e.get("bytes_per_launch")


def make_inputs(torch, synth, n, dev, grad):
    import numpy as np
    x = torch.empty((n, 4, 5120), dtype=torch.bfloat16, device=dev)
    kv = torch.empty((n, 25600), dtype=torch.bfloat16, device=dev)
    m = torch.empty(n, dtype=torch.uint8, device=dev)
    synth.dev_normal_bf16(x, SEED, synth.ID_X)
    synth.dev_normal_bf16(kv, SEED, synth.ID_KV)
    synth.dev_mask(m, SEED, P_MASK)
    w = torch.from_numpy(synth.normal_f32(4 * 5120, SEED, synth.ID_W, 1.0, 0.1).reshape(4, 5120)).to(dev)
    g = None
    if grad:
        g = torch.empty((n, 4, 5120), dtype=torch.bfloat16, device=dev)
        synth.dev_normal_bf16(g, SEED, synth.ID_GRAD)
    return x, kv, w, m, g


def host_cpu():
    """The host CPU's model name and logical CPU count (for the oracle baseline)."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "nproc": os.cpu_count()}


def cpu_baseline(seconds=10.0, sample=2048):
    """The fp64 oracle on the host cores: fwd+bwd over the first `sample`
    tokens of the same workload, repeated until `seconds` have elapsed."""
    import oracle
    import synth
    inp = synth.host_inputs(sample, seed=SEED, p=P_MASK, grad=True)
    threads = oracle.default_threads()
    # one untimed pass touches every page of the outputs
    oracle.fwd_bf16(inp["x"][:8], inp["kv"][:8], inp["weight"], inp["mask"][:8], threads=threads)
    done = 0
    t0 = time.perf_counter()
    while True:
        _, saved = oracle.fwd_bf16(inp["x"], inp["kv"], inp["weight"], inp["mask"], threads=threads)
        oracle.bwd_bf16(inp["x"], inp["kv"], inp["weight"], saved, inp["grad_out"], threads=threads)
        done += sample
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    res = {"value": done / el, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"fwd+bwd on the first {sample} tokens of the N={N_STEP} workload, "
                     f"repeated {done // sample}x over {el:.1f} s (fp64, {threads} threads)"}
    # the same on one thread, over a smaller sample
    one = inp["x"][:256], inp["kv"][:256], inp["mask"][:256], inp["grad_out"][:256]
    done1, t1 = 0, time.perf_counter()
    while True:
        _, sv1 = oracle.fwd_bf16(one[0], one[1], inp["weight"], one[2], threads=1)
        oracle.bwd_bf16(one[0], one[1], inp["weight"], sv1, one[3], threads=1)
        done1 += 256
        el1 = time.perf_counter() - t1
        if el1 >= seconds / 4:
            break
    res["single_thread"] = {"value": done1 / el1, "unit": "tokens/s", "cores": 1,
                            "sample": f"fwd+bwd on the first 256 tokens, repeated {done1 // 256}x over {el1:.1f} s"}
    res["host"] = host_cpu()
    return res


def bench_gateconv(torch, synth, eg, dev, stream, steps, R):
    """GateConv forward then backward over M x T x d, R rotated buffer sets;
    HIP events around each call on the launching stream."""
    M, T, d = GC_M, GC_T, GC_D
    sets = []
    for _ in range(R):
        b = {}
        for name, tid in (("H", synth.ID_GC_H), ("k", synth.ID_GC_K), ("v", synth.ID_GC_V), ("dY", synth.ID_GC_DY)):
            b[name] = torch.empty((M, T, d), dtype=torch.bfloat16, device=dev)
            synth.dev_normal_bf16(b[name], SEED, tid)
        b["wh"] = torch.from_numpy(synth.normal_f32(d, SEED, synth.ID_GC_WH, 1.0, 0.25)).to(dev)
        b["wv"] = torch.from_numpy(synth.normal_f32(d, SEED, synth.ID_GC_WV, 1.0, 0.25)).to(dev)
        b["cw"] = torch.from_numpy(synth.normal_f32(4 * d, SEED, synth.ID_GC_CW, 0.0, 0.5).reshape(4, d)).to(dev)
        for name in ("Y", "vhat", "dH", "dk", "dv"):
            b[name] = torch.empty((M, T, d), dtype=torch.bfloat16, device=dev)
        for name in ("alpha", "rh", "rk", "rv"):
            b[name] = torch.empty((M, T), dtype=torch.float32, device=dev)
        for name in ("dwh", "dwv"):
            b[name] = torch.empty(d, dtype=torch.float32, device=dev)
        b["dcw"] = torch.empty((4, d), dtype=torch.float32, device=dev)
        b["ws"] = torch.empty(eg.engram_gateconv_bwd_workspace_bytes(M, T, d), dtype=torch.uint8, device=dev)
        sets.append(b)

    def fwd(b):
        eg.engram_gateconv_fwd(b["H"], b["k"], b["v"], b["wh"], b["wv"], b["cw"], b["Y"], b["vhat"], b["alpha"],
                               b["rh"], b["rk"], b["rv"], stream=stream)

    def bwd(b):
        eg.engram_gateconv_bwd(b["dY"], b["H"], b["k"], b["v"], b["wh"], b["wv"], b["cw"], b["vhat"], b["alpha"],
                               b["rh"], b["rk"], b["rv"], b["dH"], b["dk"], b["dv"], b["dwh"], b["dwv"], b["dcw"],
                               b["ws"], stream=stream)

    for i in range(5):
        fwd(sets[i % R])
        bwd(sets[i % R])
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        b = sets[i % R]
        ev[i][0].record(stream)
        fwd(b)
        ev[i][1].record(stream)
        bwd(b)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    f_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    b_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    fb, bb = gc_fwd_bytes(M, T, d), gc_bwd_bytes(M, T, d)
    f_gbps, b_gbps = fb / (f_ms * 1e-3) / 1e9, bb / (b_ms * 1e-3) / 1e9
    sets.clear()
    torch.cuda.empty_cache()
    return {"workload": f"TileOPs GateConv fwd+bwd, M={M} sequences x T={T} tokens x d={d} (bf16 H/k/v/dY "
                        f"N(0,1), fp32 rms_w N(1,0.25^2), conv_w N(0,0.5^2), seed {SEED})",
            "tokens_per_s": round(M * T / ((f_ms + b_ms) * 1e-3), 1),
            "fwd": {"us": round(f_ms * 1e3, 2), "tensor_gbps": round(f_gbps, 1),
                    "frac_of_peak": round(f_gbps / PEAK_GBPS, 4), "algorithmic_bytes_per_launch": fb,
                    "traffic": recorded_traffic("gc_fwd")},
            "bwd": {"us": round(b_ms * 1e3, 2), "tensor_gbps": round(b_gbps, 1),
                    "frac_of_peak": round(b_gbps / PEAK_GBPS, 4), "algorithmic_bytes_per_launch": bb,
                    "traffic": recorded_traffic("gc_bwd"),
                    "kernels": "gateconv_bwd_conv_kernel + gateconv_bwd_hk_kernel + gateconv_reduce_kernel"},
            "steps": steps, "buffer_sets_rotated": R}


# The five workload configurations: forward N=64; forward N=8192; forward +
# backward N=4096; forward N=1,048,512 in one launch; forward + backward at
# N=8192 with mask Bernoulli(0.3) and the edge-row recipe (5% of rows with X
# or a key scaled by 1e-12, 10% of dots inside the clamp), 1000 launches.
CONFIGS = [
    dict(config=0, op="fwd", tokens=64, mask_p=0.9, edge=False, launches=200,
         desc="forward, N=64, mask Bernoulli(0.9)"),
    dict(config=1, op="fwd", tokens=8192, mask_p=0.9, edge=False, launches=200,
         desc="forward, N=8192, mask Bernoulli(0.9)"),
    dict(config=2, op="fwd+bwd", tokens=4096, mask_p=0.9, edge=False, launches=200,
         desc="forward + backward, N=4096, mask Bernoulli(0.9), grad_out N(0,1)"),
    dict(config=3, op="fwd", tokens=N_LARGE, mask_p=0.9, edge=False, launches=5,
         desc="forward, N=1,048,512 in one launch (~140 GB resident), mask Bernoulli(0.9)"),
    dict(config=4, op="fwd+bwd", tokens=8192, mask_p=0.3, edge=True, launches=1000,
         desc="forward + backward, N=8192, mask Bernoulli(0.3), eps/clamp/zero edge rows, "
              "1000 launches back to back on one stream"),
]


def recorded_config_traffic(config):
    """HBM bytes per call of a configuration from the rocprofv3 counter runs,
    if taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    e = rec.get("configs", {}).get(str(config))
    if not e or e.get("source_hash") != kernel_source_hash("bwd" if CONFIGS[config]["op"] != "fwd" else "fwd"):
        return None
    return e.get("bytes_per_call")


def oracle_rate(op, n, p, edge, seconds=3.0, sample=2048):
    """The fp64 oracle on the host cores over the first min(n, sample) tokens
    of a configuration's workload, repeated for about `seconds`."""
    import oracle
    import synth
    nt = min(n, sample)
    inp = synth.host_inputs(n, seed=SEED, p=p, nt=nt, grad=op != "fwd", edge=edge)
    threads = oracle.default_threads()
    oracle.fwd_bf16(inp["x"][:8], inp["kv"][:8], inp["weight"], inp["mask"][:8], threads=threads)
    done, t0 = 0, time.perf_counter()
    while True:
        _, saved = oracle.fwd_bf16(inp["x"], inp["kv"], inp["weight"], inp["mask"], threads=threads)
        if op != "fwd":
            oracle.bwd_bf16(inp["x"], inp["kv"], inp["weight"], saved, inp["grad_out"], threads=threads)
        done += nt
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"tokens_per_s": round(done / el, 1), "cores": threads,
            "sample": f"{op} on the first {nt} tokens, repeated {done // nt}x over {el:.1f} s (fp64)"}


def measure_config(torch, synth, eg, dev, stream, c, rotate):
    """One workload configuration on the GPU: time per call (the configuration's
    launches back to back on the launch stream, between two HIP events, over
    their count), tokens/s, tensor-byte GB/s and its fraction of 8 TB/s; below
    1000 launches also the median of single calls, each between two events of
    its own (each recorded event holds the stream a few microseconds, which
    the back-to-back time leaves out).  Configurations 0-2 cycle `rotate`
    independent buffer sets (so no call finds its inputs in the 256 MB cache);
    configuration 3 has one set (140 GB); configuration 4 repeats its 1000
    launches on one set, as specified."""
    n, op = c["tokens"], c["op"]
    grad = op != "fwd"
    R = rotate if c["config"] <= 2 else 1
    sets = []
    for _ in range(R):
        if c["edge"]:
            h = synth.host_inputs(n, seed=SEED, p=c["mask_p"], grad=grad, edge=True)
            x = torch.from_numpy(h["x"].view("int16")).view(torch.bfloat16).to(dev)
            kv = torch.from_numpy(h["kv"].view("int16")).view(torch.bfloat16).to(dev)
            w = torch.from_numpy(h["weight"]).to(dev)
            m = torch.from_numpy(h["mask"]).to(dev)
            g = torch.from_numpy(h["grad_out"].view("int16")).view(torch.bfloat16).to(dev) if grad else None
            del h
        else:
            x = torch.empty((n, 4, 5120), dtype=torch.bfloat16, device=dev)
            kv = torch.empty((n, 25600), dtype=torch.bfloat16, device=dev)
            m = torch.empty(n, dtype=torch.uint8, device=dev)
            synth.dev_normal_bf16(x, SEED, synth.ID_X)
            synth.dev_normal_bf16(kv, SEED, synth.ID_KV)
            synth.dev_mask(m, SEED, c["mask_p"])
            w = torch.from_numpy(synth.normal_f32(4 * 5120, SEED, synth.ID_W, 1.0, 0.1).reshape(4, 5120)).to(dev)
            g = None
            if grad:
                g = torch.empty((n, 4, 5120), dtype=torch.bfloat16, device=dev)
                synth.dev_normal_bf16(g, SEED, synth.ID_GRAD)
        b = dict(x=x, kv=kv, w=w, m=m, g=g, out=torch.empty_like(x),
                 saved=torch.empty((n, 4, 4), dtype=torch.float32, device=dev))
        if grad:
            b.update(gx=torch.empty_like(x), gkv=torch.empty_like(kv),
                     gw=torch.empty((4, 5120), dtype=torch.float32, device=dev),
                     ws=torch.empty(eg.engram_gate_bwd_workspace_bytes(n), dtype=torch.uint8, device=dev))
        sets.append(b)
        x = kv = w = m = g = None

    def call(b):
        eg.engram_gate_fwd(b["x"], b["kv"], b["w"], b["m"], b["out"], b["saved"], n, stream=stream)
        if grad:
            eg.engram_gate_bwd(b["x"], b["kv"], b["w"], b["saved"], b["g"], b["gx"], b["gkv"], b["gw"],
                               b["ws"], n, stream=stream)

    for i in range(max(3, R)):
        call(sets[i % R])
    torch.cuda.synchronize()
    K = c["launches"]
    # the calls back to back on one stream: the time of the K calls over K
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(K):
        call(sets[i % R])
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / K
    us_median = None
    if K < 1000:  # also the median of single calls, each between two events of its own
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(K)]
        for i, (a, z) in enumerate(ev):
            a.record(stream)
            call(sets[i % R])
            z.record(stream)
        torch.cuda.synchronize()
        us_median = sorted(a.elapsed_time(z) for a, z in ev)[K // 2] * 1e3
    byt = fwd_bytes(n) + (bwd_bytes(n) if grad else 0)
    gbps = byt / (us * 1e-6) / 1e9
    sets.clear()
    torch.cuda.empty_cache()
    line = {"config": c["config"], "workload": c["desc"], "op": op, "tokens": n, "mask_p": c["mask_p"],
            "edge_rows": c["edge"], "launches": K, "buffer_sets_rotated": R, "us_per_call": round(us, 2),
            "us_per_call_timing": "K calls back to back on one stream, over K",
            "tokens_per_s": round(n / (us * 1e-6), 1), "tensor_bytes_per_call": byt,
            "tensor_gbps": round(gbps, 1), "frac_of_peak_tensor_bytes": round(gbps / PEAK_GBPS, 4)}
    if us_median is not None:
        line["us_median_single_call"] = round(us_median, 2)
    moved = recorded_config_traffic(c["config"])
    if moved:
        # the HBM bytes a call actually moves (the backward skips reads where delta is 0)
        line["traffic_bytes_per_call"] = moved
        line["traffic_gbps"] = round(moved / (us * 1e-6) / 1e9, 1)
        line["frac_of_peak_traffic"] = round(moved / (us * 1e-6) / 1e9 / PEAK_GBPS, 4)
    return line


SWEEP_FWD = (64, 256, 1024, 2048, 4096, 8192, 32768, 131072, 524288, N_LARGE)
SWEEP_STEP = (64, 256, 1024, 2048, 4096, 8192)


def bench_sweep(torch, synth, eg, dev, stream, rotate):
    """Throughput against the token count: the forward alone, and forward +
    backward (the backward's accepted sizes), each timed as in
    measure_config (calls back to back, rotating buffer sets while they fit
    in about 100 GB); one JSON line per size."""
    # device bytes of one buffer set per token: inputs and outputs (the backward's
    # grad_out, grad_x and grad_kv on top of the forward's)
    per_token = {"fwd": fwd_bytes(1) + 40960 + 64, "fwd+bwd": fwd_bytes(1) + bwd_bytes(1) + 3 * 40960 + 51200}
    for op, sizes in (("fwd", SWEEP_FWD), ("fwd+bwd", SWEEP_STEP)):
        for n in sizes:
            fit = max(1, int(100e9 // (per_token[op] * n)))
            c = dict(config=-1, op=op, tokens=n, mask_p=0.9, edge=False,
                     # about 0.2 s of calls at 6 TB/s, 5 to 200 of them
                     launches=max(5, min(200, int(1.2e12 // (fwd_bytes(n) + (bwd_bytes(n) if op != "fwd" else 0))))),
                     desc=f"{op}, N={n}, mask Bernoulli(0.9)")
            line = measure_config(torch, synth, eg, dev, stream, c, min(rotate, fit))
            line.pop("config")
            print(json.dumps(line), flush=True)


def bench_configs(torch, synth, eg, dev, stream, with_cpu, rotate):
    """One JSON line per configuration (measure_config), with the oracle's
    rate on a bounded sample beside it."""
    for c in CONFIGS:
        line = measure_config(torch, synth, eg, dev, stream, c, rotate)
        if with_cpu:
            line["oracle"] = oracle_rate(c["op"], c["tokens"], c["mask_p"], c["edge"])
            line["oracle"]["host"] = host_cpu()
            line["speedup_vs_oracle"] = round(line["tokens_per_s"] / line["oracle"]["tokens_per_s"], 1)
        print(json.dumps(line), flush=True)


def bench_placement(torch, synth, eg, dev, stream, reps=5):
    """The N = 1,048,512 forward (one launch, ~140 GB) under several placements
    of its three large tensors, in one process: X, KV and out allocated
    separately in each of three orders, and carved from one allocation.  The
    caching allocator is emptied between placements so each gets fresh device
    memory.  Prints one JSON line per placement (median of `reps` launches)."""
    nl = N_LARGE
    shapes = {"x": ((nl, 4, 5120), torch.bfloat16), "kv": ((nl, 25600), torch.bfloat16),
              "out": ((nl, 4, 5120), torch.bfloat16)}
    orders = [("x", "kv", "out"), ("kv", "out", "x"), ("out", "x", "kv"), "pooled"]
    w = torch.from_numpy(synth.normal_f32(4 * 5120, SEED, synth.ID_W, 1.0, 0.1).reshape(4, 5120)).to(dev)
    m = torch.empty(nl, dtype=torch.uint8, device=dev)
    synth.dev_mask(m, SEED, P_MASK)
    saved = torch.empty((nl, 4, 4), dtype=torch.float32, device=dev)
    for order in orders:
        torch.cuda.empty_cache()
        t = {}
        if order == "pooled":
            sizes = {k: int(torch.Size(sh).numel()) for k, (sh, _) in shapes.items()}
            pool = torch.empty(sum(sizes.values()), dtype=torch.bfloat16, device=dev)
            off = 0
            for k in ("x", "kv", "out"):
                t[k] = pool[off:off + sizes[k]].view(shapes[k][0])
                off += sizes[k]
        else:
            for k in order:
                t[k] = torch.empty(shapes[k][0], dtype=shapes[k][1], device=dev)
        synth.dev_normal_bf16(t["x"], SEED, synth.ID_X)
        synth.dev_normal_bf16(t["kv"], SEED, synth.ID_KV)
        for _ in range(2):
            eg.engram_gate_fwd(t["x"], t["kv"], w, m, t["out"], saved, nl, stream=stream)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for i in range(reps):
            ev[i][0].record(stream)
            eg.engram_gate_fwd(t["x"], t["kv"], w, m, t["out"], saved, nl, stream=stream)
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        ms = sorted(e[0].elapsed_time(e[1]) for e in ev)
        gbps = fwd_bytes(nl) / (ms[reps // 2] * 1e-3) / 1e9
        print(json.dumps({"placement": order if order == "pooled" else "separate, allocated " + ", ".join(order),
                          "addresses": {k: hex(v.data_ptr()) for k, v in t.items()},
                          "ms_median": round(ms[reps // 2], 3), "ms_all": [round(x, 3) for x in ms],
                          "tensor_gbps": round(gbps, 1), "frac_of_peak": round(gbps / PEAK_GBPS, 4)}), flush=True)
        t.clear()
        pool = None


def bench_same_buffers(torch, synth, eg, dev, stream, placements=3, reps=20, sets_per_placement=5):
    """The gate's kernels against plain streams of exactly their traffic, over
    the same buffers in the same process (the probe library's kernels: whole
    tokens per 512-thread workgroup in lockstep over 256 or 1024 workgroups,
    and the backward's own split -- a quarter of every row per 256-thread
    workgroup).  Each placement allocates `sets_per_placement` fresh buffer
    sets of the N = 8192 step.  Two contexts, medians of `reps` calls each:
      cold: every call runs on a different buffer set than the call before it,
        so none reads what the previous call left in the 256 MB last-level
        cache (back-to-back calls on the same buffers gain up to ~15% from it,
        by an amount that depends on the order of both calls);
      after_fwd: the gate's forward on a set, then the timed call on the same
        set -- the benchmark step's context for the backward.
    One JSON line per placement."""
    import ctypes
    plib = ctypes.CDLL(os.path.join(ROOT, "memory_bound_engram_amd", "probe", "libengram_probe.so"))
    plib.probe_stream.argtypes = [ctypes.c_char_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_void_p]
    plib.probe_stream.restype = ctypes.c_int
    n = N_STEP
    stream_fwd_bytes = (40960 + 51200 + 40960) * n
    stream_bwd_bytes = (40960 + 51200 + 40960 + 40960 + 51200) * n

    def probe(shape, ins, outs, grid, deal):
        a_in = (ctypes.c_void_p * len(ins))(*[t.data_ptr() for t in ins])
        a_out = (ctypes.c_void_p * len(outs))(*[t.data_ptr() for t in outs])
        rc = plib.probe_stream(shape.encode(), a_in, a_out, n, grid, deal, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"probe_stream({shape}) returned {rc}")

    def sfwd(grid):
        return lambda b: probe("fwd", [b["x"], b["kv"]], [b["out"]], grid, 0)

    def sbwd(grid, deal):
        return lambda b: probe("bwd", [b["x"], b["kv"], b["g"]], [b["gx"], b["gkv"]], grid, deal)

    gate_fwd = lambda b: eg.engram_gate_fwd(b["x"], b["kv"], b["w"], b["m"], b["out"], b["saved"], n, stream=stream)
    gate_bwd = lambda b: eg.engram_gate_bwd(b["x"], b["kv"], b["w"], b["saved"], b["g"], b["gx"], b["gkv"], b["gw"],
                                            b["ws"], n, stream=stream)
    calls = {"gate_fwd": gate_fwd, "stream_fwd_lockstep256": sfwd(256), "stream_fwd_lockstep1024": sfwd(1024),
             "gate_bwd": gate_bwd, "stream_bwd_lockstep256": sbwd(256, 0), "stream_bwd_lockstep1024": sbwd(1024, 0),
             "stream_bwd_quarters4096": sbwd(4096, 3)}
    after = ["gate_bwd", "stream_bwd_lockstep256", "stream_bwd_lockstep1024"]
    own = {"gate_fwd": fwd_bytes(n), "gate_bwd": bwd_bytes(n)}

    def timed(f, b, pre=None):
        if pre is not None:
            pre(b)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        f(b)
        e1.record(stream)
        return e0, e1

    def medians(ev):
        return {k: round(sorted(a.elapsed_time(z) for a, z in v)[len(v) // 2] * 1e3, 2) for k, v in ev.items()}

    for pl in range(placements):
        torch.cuda.empty_cache()
        sets = []
        for _ in range(sets_per_placement):
            x, kv, w, m, g = make_inputs(torch, synth, n, dev, grad=True)
            sets.append(dict(x=x, kv=kv, w=w, m=m, g=g, out=torch.empty_like(x),
                             saved=torch.empty((n, 4, 4), dtype=torch.float32, device=dev),
                             gx=torch.empty_like(x), gkv=torch.empty_like(kv),
                             gw=torch.empty((4, 5120), dtype=torch.float32, device=dev),
                             ws=torch.empty(eg.engram_gate_bwd_workspace_bytes(n), dtype=torch.uint8, device=dev)))
        for b in sets:  # the backward needs the forward's saved state
            gate_fwd(b)
        c = 0  # call counter: call c runs on set c mod R, never the previous call's set
        R = len(sets)
        cold = {k: [] for k in calls}
        for i in range(2 + reps):
            for k, f in calls.items():
                pair = timed(f, sets[c % R])
                c += 1
                if i >= 2:
                    cold[k].append(pair)
        post = {k: [] for k in after}
        for i in range(2 + reps):
            for k in after:
                pair = timed(calls[k], sets[c % R], pre=gate_fwd)
                c += 1
                if i >= 2:
                    post[k].append(pair)
        torch.cuda.synchronize()
        us_cold, us_after = medians(cold), medians(post)

        def rate(k, v):
            return round((own.get(k) or (stream_fwd_bytes if "fwd" in k else stream_bwd_bytes)) / (v * 1e-6) / 1e12, 3)

        best_fwd = min(v for k, v in us_cold.items() if k.startswith("stream_fwd"))
        best_bwd = min(v for k, v in us_cold.items() if k.startswith("stream_bwd"))
        best_bwd_after = min(v for k, v in us_after.items() if k.startswith("stream_bwd"))
        line = {"placement": pl, "tokens": n, "buffer_sets": R, "reps": reps,
                "cold_us": us_cold, "cold_tb_s_own_bytes": {k: rate(k, v) for k, v in us_cold.items()},
                "after_fwd_us": us_after,
                "gate_fwd_vs_best_stream_cold": round(best_fwd / us_cold["gate_fwd"], 4),
                "gate_bwd_vs_best_stream_cold": round(best_bwd / us_cold["gate_bwd"], 4),
                "gate_bwd_vs_best_stream_after_fwd": round(best_bwd_after / us_after["gate_bwd"], 4)}
        print(json.dumps(line), flush=True)
        sets.clear()


def bench_same_buffers_gateconv(torch, synth, eg, dev, stream, placements=3, reps=20, sets_per_placement=5):
    """GateConv's kernels against plain streams of exactly their traffic over
    the same buffers (M = 4 x T = 4096 rows at d = 5120), timed cold as in
    bench_same_buffers: every call on a different buffer set than the call
    before it.  The streams (the probe library's, 512-thread workgroups, a row
    of every tensor per workgroup and step) deal the rows either in chunks of
    consecutive rows, as GateConv's kernels must for the conv history (256
    workgroups of 64 rows), or round-robin (lockstep).  One JSON line per
    placement."""
    import ctypes
    plib = ctypes.CDLL(os.path.join(ROOT, "memory_bound_engram_amd", "probe", "libengram_probe.so"))
    plib.probe_stream.argtypes = [ctypes.c_char_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_void_p]
    plib.probe_stream.restype = ctypes.c_int
    M, T, d = GC_M, GC_T, GC_D
    rows = M * T

    def probe(shape, ins, outs, grid, deal):
        a_in = (ctypes.c_void_p * len(ins))(*[t.data_ptr() for t in ins])
        a_out = (ctypes.c_void_p * len(outs))(*[t.data_ptr() for t in outs])
        rc = plib.probe_stream(shape.encode(), a_in, a_out, rows, grid, deal, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"probe_stream({shape}) returned {rc}")

    def fwd(b):
        eg.engram_gateconv_fwd(b["H"], b["k"], b["v"], b["wh"], b["wv"], b["cw"], b["Y"], b["vhat"], b["alpha"],
                               b["rh"], b["rk"], b["rv"], stream=stream)

    def bwd(b):
        eg.engram_gateconv_bwd(b["dY"], b["H"], b["k"], b["v"], b["wh"], b["wv"], b["cw"], b["vhat"], b["alpha"],
                               b["rh"], b["rk"], b["rv"], b["dH"], b["dk"], b["dv"], b["dwh"], b["dwv"], b["dcw"],
                               b["ws"], stream=stream)

    def sfwd(grid, deal):
        return lambda b: probe("gcfwd", [b["H"], b["k"], b["v"]], [b["Y"], b["vhat"]], grid, deal)

    def sbwd(grid, deal):
        return lambda b: probe("gcbwd", [b["dY"], b["H"], b["k"], b["v"], b["vhat"]], [b["dH"], b["dk"], b["dv"]],
                               grid, deal)

    calls = {"gateconv_fwd": fwd, "stream_fwd_chunked256": sfwd(256, 1), "stream_fwd_lockstep256": sfwd(256, 0),
             "stream_fwd_lockstep1024": sfwd(1024, 0),
             "gateconv_bwd": bwd, "stream_bwd_chunked256": sbwd(256, 1), "stream_bwd_lockstep256": sbwd(256, 0),
             "stream_bwd_lockstep1024": sbwd(1024, 0)}
    own = {"gateconv_fwd": gc_fwd_bytes(M, T, d), "gateconv_bwd": gc_bwd_bytes(M, T, d)}
    stream_bytes = {"fwd": 5 * 2 * d * rows, "bwd": 8 * 2 * d * rows}
    for pl in range(placements):
        torch.cuda.empty_cache()
        sets = []
        for _ in range(sets_per_placement):
            b = {}
            for name, tid in (("H", synth.ID_GC_H), ("k", synth.ID_GC_K), ("v", synth.ID_GC_V), ("dY", synth.ID_GC_DY)):
                b[name] = torch.empty((M, T, d), dtype=torch.bfloat16, device=dev)
                synth.dev_normal_bf16(b[name], SEED, tid)
            b["wh"] = torch.from_numpy(synth.normal_f32(d, SEED, synth.ID_GC_WH, 1.0, 0.25)).to(dev)
            b["wv"] = torch.from_numpy(synth.normal_f32(d, SEED, synth.ID_GC_WV, 1.0, 0.25)).to(dev)
            b["cw"] = torch.from_numpy(synth.normal_f32(4 * d, SEED, synth.ID_GC_CW, 0.0, 0.5).reshape(4, d)).to(dev)
            for name in ("Y", "vhat", "dH", "dk", "dv"):
                b[name] = torch.empty((M, T, d), dtype=torch.bfloat16, device=dev)
            for name in ("alpha", "rh", "rk", "rv"):
                b[name] = torch.empty((M, T), dtype=torch.float32, device=dev)
            for name in ("dwh", "dwv"):
                b[name] = torch.empty(d, dtype=torch.float32, device=dev)
            b["dcw"] = torch.empty((4, d), dtype=torch.float32, device=dev)
            b["ws"] = torch.empty(eg.engram_gateconv_bwd_workspace_bytes(M, T, d), dtype=torch.uint8, device=dev)
            fwd(b)  # the backward reads the forward's saved tensors
            sets.append(b)
        R, c = len(sets), 0
        ev = {k: [] for k in calls}
        for i in range(2 + reps):
            for k, f in calls.items():
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                b = sets[c % R]
                c += 1
                e0.record(stream)
                f(b)
                e1.record(stream)
                if i >= 2:
                    ev[k].append((e0, e1))
        torch.cuda.synchronize()
        us = {k: round(sorted(a.elapsed_time(z) for a, z in v)[len(v) // 2] * 1e3, 2) for k, v in ev.items()}
        rate = {k: round((own.get(k) or stream_bytes["fwd" if "fwd" in k else "bwd"]) / (v * 1e-6) / 1e12, 3)
                for k, v in us.items()}
        line = {"placement": pl, "rows": rows, "d": d, "buffer_sets": R, "reps": reps, "cold_us": us,
                "cold_tb_s_own_bytes": rate,
                "fwd_vs_chunked_stream": round(us["stream_fwd_chunked256"] / us["gateconv_fwd"], 4),
                "fwd_vs_best_stream": round(min(v for k, v in us.items() if k.startswith("stream_fwd"))
                                            / us["gateconv_fwd"], 4),
                "bwd_vs_best_stream": round(min(v for k, v in us.items() if k.startswith("stream_bwd"))
                                            / us["gateconv_bwd"], 4)}
        print(json.dumps(line), flush=True)
        sets.clear()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-large", action="store_true", help="skip the N=1,048,512 forward")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the per-configuration timings that the benchmark line carries")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-gateconv", action="store_true", help="skip the GateConv forward/backward")
    ap.add_argument("--gateconv-steps", type=int, default=50)
    ap.add_argument("--rotate", type=int, default=4,
                    help="independent input/output sets cycled step by step, so that no step "
                         "finds its data in cache from the previous one")
    ap.add_argument("--configs", action="store_true",
                    help="instead of the benchmark line, one line per workload configuration (0-4)")
    ap.add_argument("--sweep", action="store_true",
                    help="instead of the benchmark line, throughput against N for the forward and for "
                         "forward + backward (one JSON line per size)")
    ap.add_argument("--placement", action="store_true",
                    help="instead of the benchmark line, the N=1,048,512 forward under several "
                         "placements of its tensors (one JSON line each)")
    ap.add_argument("--same-buffers", action="store_true",
                    help="instead of the benchmark line, the gate's kernels against plain streams of the "
                         "same traffic over the same buffers (cold, and the backward after the forward), "
                         "for three fresh placements")
    ap.add_argument("--same-buffers-gateconv", action="store_true",
                    help="instead of the benchmark line, GateConv's kernels against plain streams of the same "
                         "traffic over the same buffers, timed cold, for three fresh placements")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run a plain 1 GiB device-to-device copy (the reference kernel that "
                         "scales rocprofv3 FETCH_SIZE/WRITE_SIZE readings)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the Engram gate is independent per token, and this "
              "build has no multi-GPU path (see the sharding notes); run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import memory_bound_engram_amd as eg

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.same_buffers:
        bench_same_buffers(torch, synth, eg, dev, torch.cuda.current_stream(dev))
        return
    if args.same_buffers_gateconv:
        bench_same_buffers_gateconv(torch, synth, eg, dev, torch.cuda.current_stream(dev))
        return
    if args.placement:
        bench_placement(torch, synth, eg, dev, torch.cuda.current_stream(dev))
        return
    if args.sweep:
        bench_sweep(torch, synth, eg, dev, torch.cuda.current_stream(dev), max(1, args.rotate))
        return
    if args.configs:
        bench_configs(torch, synth, eg, dev, torch.cuda.current_stream(dev), not args.no_cpu, max(1, args.rotate))
        return
    n = N_STEP
    R = max(1, args.rotate)
    sets = []
    for _ in range(R):  # same seeded data, distinct memory
        x, kv, w, m, g = make_inputs(torch, synth, n, dev, grad=True)
        sets.append(dict(x=x, kv=kv, w=w, m=m, g=g, out=torch.empty_like(x),
                         saved=torch.empty((n, 4, 4), dtype=torch.float32, device=dev),
                         gx=torch.empty_like(x), gkv=torch.empty_like(kv),
                         gw=torch.empty((4, 5120), dtype=torch.float32, device=dev),
                         ws=torch.empty(eg.engram_gate_bwd_workspace_bytes(n), dtype=torch.uint8, device=dev)))
    stream = torch.cuda.current_stream(dev)

    def fwd(b):
        eg.engram_gate_fwd(b["x"], b["kv"], b["w"], b["m"], b["out"], b["saved"], n, stream=stream)

    def bwd(b):
        eg.engram_gate_bwd(b["x"], b["kv"], b["w"], b["saved"], b["g"], b["gx"], b["gkv"], b["gw"], b["ws"], n,
                           stream=stream)

    for i in range(args.warmup):
        fwd(sets[i % R])
        bwd(sets[i % R])
    torch.cuda.synchronize()

    K = args.steps
    # the step rate: K steps back to back with nothing else on the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        b = sets[i % R]
        fwd(b)
        bwd(b)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # per-call durations: a second pass of the same K steps with HIP events
    # around each call on the launch stream.  Each recorded event holds the
    # stream for a few microseconds between calls (about 10 us a step here),
    # so the events stay out of the pass that gives the rate.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for i in range(K):
        b = sets[i % R]
        ev[i][0].record(stream)
        fwd(b)
        ev[i][1].record(stream)
        bwd(b)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    elapsed_with_events = time.perf_counter() - t1
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / K
    bwd_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / K

    fwd_gbps = fwd_bytes(n) / (fwd_ms * 1e-3) / 1e9
    bwd_gbps = bwd_bytes(n) / (bwd_ms * 1e-3) / 1e9
    both_gbps = (fwd_bytes(n) + bwd_bytes(n)) / ((fwd_ms + bwd_ms) * 1e-3) / 1e9
    step_gbps = (fwd_bytes(n) + bwd_bytes(n)) / (elapsed / K) / 1e9
    dominant = "bwd" if bwd_ms >= fwd_ms else "fwd"
    if dominant == "bwd":
        roof = {"kernel": "engram_gate_bwd (main kernel + grad_weight column reduce)",
                "bound": "hbm", "achieved": round(bwd_gbps, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                "frac": round(bwd_gbps / PEAK_GBPS, 4), "launch_us": round(bwd_ms * 1e3, 2),
                "algorithmic_bytes_per_launch": bwd_bytes(n),
                "traffic": recorded_traffic("bwd")}
    else:
        roof = {"kernel": "engram_fwd_kernel", "bound": "hbm", "achieved": round(fwd_gbps, 1),
                "peak": PEAK_GBPS, "unit": "GB/s", "frac": round(fwd_gbps / PEAK_GBPS, 4),
                "launch_us": round(fwd_ms * 1e3, 2), "algorithmic_bytes_per_launch": fwd_bytes(n),
                "traffic": recorded_traffic("fwd")}
    # the HBM bytes the launch actually moves (masked tokens skip reads), over the same time
    if roof["traffic"]:
        roof["traffic_gbps"] = round(roof["traffic"] / (roof["launch_us"] * 1e-6) / 1e9, 1)

    res = {
        "metric": METRIC,
        "value": round(n * K / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / K * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "engram gate fwd+bwd, N=8192 tokens x 4 streams x 5120 (bf16 X/KV/grads, "
                               "fp32 weight/saved), mask Bernoulli(0.9), grad_out N(0,1), seed 0",
                   "inputs_of_config": 1, "size_and_ops_of_config": 4,
                   "tokens": n, "streams": 4, "hidden": 5120, "mask_p": P_MASK, "buffer_sets_rotated": R},
        "fwd": {"tokens_per_s": round(n / (fwd_ms * 1e-3), 1), "us": round(fwd_ms * 1e3, 2),
                "tensor_gbps": round(fwd_gbps, 1), "frac_of_peak": round(fwd_gbps / PEAK_GBPS, 4)},
        "bwd": {"tokens_per_s": round(n / (bwd_ms * 1e-3), 1), "us": round(bwd_ms * 1e3, 2),
                "tensor_gbps": round(bwd_gbps, 1), "frac_of_peak": round(bwd_gbps / PEAK_GBPS, 4)},
        "fwd_bwd": {"tokens_per_s": round(n / ((fwd_ms + bwd_ms) * 1e-3), 1),
                    "tensor_gbps": round(both_gbps, 1), "frac_of_peak": round(both_gbps / PEAK_GBPS, 4)},
        "step": {"us": round(elapsed / K * 1e6, 2), "tensor_gbps": round(step_gbps, 1),
                 "frac_of_peak": round(step_gbps / PEAK_GBPS, 4),
                 "us_with_per_call_events": round(elapsed_with_events / K * 1e6, 2),
                 "timing": "value and ms_per_step: K steps back to back, no per-call events; fwd, bwd, "
                           "fwd_bwd and roofline: a second pass of the K steps with HIP events around each call"},
        "roofline": roof,
    }
    sets.clear()
    x = kv = w = m = g = b = None
    torch.cuda.empty_cache()

    if not args.no_configs:
        # every workload configuration, timed on the GPU (no oracle leg here)
        res["configs"] = {}
        for c in CONFIGS:
            if c["tokens"] == N_LARGE:
                free, _ = torch.cuda.mem_get_info(dev)
                if args.no_large or free <= N_LARGE * (2 * 40960 + 51200 + 65) + (2 << 30):
                    res["configs"][str(c["config"])] = {"config": c["config"], "workload": c["desc"],
                                                        "skipped": "--no-large" if args.no_large else
                                                        "needs ~140 GB free device memory"}
                    continue
            res["configs"][str(c["config"])] = measure_config(torch, synth, eg, dev, stream, c, R)
        big = res["configs"].get("3", {})
        if "us_per_call" in big:  # the single 140 GB launch, under its earlier name as well
            res["fwd_large"] = {"tokens": N_LARGE, "tokens_per_s": big["tokens_per_s"],
                                "ms": round(big["us_per_call"] * 1e-3, 3), "tensor_gbps": big["tensor_gbps"],
                                "frac_of_peak": big["frac_of_peak_tensor_bytes"]}

    if not args.no_gateconv:
        res["gateconv"] = bench_gateconv(torch, synth, eg, dev, stream, args.gateconv_steps, R)

    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
