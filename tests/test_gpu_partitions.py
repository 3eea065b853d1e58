"""The kernels' work partition is invisible in their results (GPU).

Each kernel deals its work out by the call's size: the forward strides a
grid over the tokens, the backward cuts them into N/64 rows of 64 tokens or
64 rows of N/64, GateConv cuts the rows into chunks whose length depends on
M T and recomputes a 3-row halo at each chunk start.  A token's (or a row's)
arithmetic does not depend on that dealing, so a call over the first n
tokens must reproduce, bit for bit, the first n tokens of a call over all of
them; outputs are pre-filled with all-ones bytes, so an element a call fails
to write, or writes beyond its size, shows up too:

  - gate forward, every n in 1..130 and sizes around each power of two up to
    8192: out and saved equal the N = 8192 call's prefix, nothing past n
    written ("Engram saved-state gate", layout paragraph: any N);
  - gate backward, every accepted n (all 128 multiples of 64 up to 8192):
    grad_x and grad_kv equal the N = 8192 call's prefix, nothing past n
    written; grad_weight (summed in another grouping) against the oracle's
    sums of 64-token blocks within the backward's grad_weight bar;
  - GateConv forward (causal: row t sees rows <= t of its sequence), the
    first T' rows of every sequence for T' from 1 to T - 1 at three widths:
    every output equals the full call's rows bit for bit ("Engram Operators",
    GateConv section).
All comparisons of large tensors run on the device.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu

D = 5120
FULL = 8192
FWD_SIZES = sorted(set(range(1, 131)) | {p + e for p in (256, 512, 1024, 2048, 4096) for e in (-1, 0, 1)}
                   | {8191, 8127, 6000})


def _poisoned_tail(t, n):
    import torch
    tail = t[n:].contiguous().view(torch.uint8)
    return bool((tail == 255).all().item())


def _same(a, b):
    import torch
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def test_fwd_prefixes(gpu):
    import torch
    from gpu_util import dev_inputs, run_fwd
    inp = synth.host_inputs(FULL, seed=51, p=0.9, edge=True)
    d = dev_inputs(inp, gpu)
    ref_out, ref_sv = run_fwd(d)
    torch.cuda.synchronize()
    bad = []
    for n in FWD_SIZES:
        out, sv = run_fwd(d, n=n)
        torch.cuda.synchronize()
        if not (_same(out[:n], ref_out[:n]) and _same(sv[:n], ref_sv[:n])
                and _poisoned_tail(out, n) and _poisoned_tail(sv, n)):
            bad.append(n)
    assert not bad, f"forward prefixes differ at n = {bad}"


def test_bwd_prefixes_every_accepted_n(gpu):
    import torch
    from gpu_util import dev_inputs, f32, run_bwd, run_fwd
    inp = synth.host_inputs(FULL, seed=52, p=0.9, grad=True, edge=True)
    d = dev_inputs(inp, gpu)
    _, saved = run_fwd(d)
    ref_gx, ref_gkv, _ = run_bwd(d, saved)
    torch.cuda.synchronize()
    sv_host = f32(saved)
    # the oracle's grad_weight per 64-token block (fp64) and its magnitude C
    blocks = []
    for b in range(FULL // 64):
        t = slice(64 * b, 64 * b + 64)
        r = oracle.bwd_bf16(inp["x"][t], inp["kv"][t], inp["weight"], sv_host[t], inp["grad_out"][t],
                            threads=8, extras=True)
        blocks.append((r[5], r[8]))
    dw64 = np.cumsum(np.stack([b[0] for b in blocks]), axis=0)
    mdw = np.cumsum(np.stack([b[1] for b in blocks]), axis=0)
    bad, worst = [], 0.0
    for k in range(1, FULL // 64 + 1):
        n = 64 * k
        gx, gkv, gw = run_bwd(d, saved, n=n)
        torch.cuda.synchronize()
        if not (_same(gx[:n], ref_gx[:n]) and _same(gkv[:n], ref_gkv[:n])
                and _poisoned_tail(gx, n) and _poisoned_tail(gkv, n)):
            bad.append(n)
        err = np.abs(f32(gw).astype(np.float64) - dw64[k - 1])
        bar = 1e-3 * np.abs(dw64[k - 1]) + 1e-4 + 2.0 ** -20 * mdw[k - 1]
        assert np.all(err <= bar), f"grad_weight at n = {n}: {np.count_nonzero(err > bar)} elements over the bar"
        worst = max(worst, float(np.max(err / bar)))
    assert not bad, f"backward prefixes differ at n = {bad}"
    print(f"grad_weight: largest error / bar over all 128 sizes {worst:.3f}")


@pytest.mark.parametrize("M,T,d", [(3, 1500, 5120), (2, 1200, 1536), (4, 700, 512)])
def test_gateconv_fwd_prefixes(gpu, M, T, d):
    import torch
    from test_gpu_gateconv import dev, empty_bf16, empty_f32
    import memory_bound_engram_amd as eg
    inp = synth.gateconv_inputs(M, T, d, seed=53, edge=True)
    H, k, v = dev(inp["H"], gpu), dev(inp["k"], gpu), dev(inp["v"], gpu)
    wh, wv, cw = dev(inp["wh"], gpu), dev(inp["wv"], gpu), dev(inp["cw"], gpu)

    def fwd(Tp):
        args = [x[:, :Tp].contiguous() for x in (H, k, v)]
        Y, vh = empty_bf16((M, Tp, d), gpu), empty_bf16((M, Tp, d), gpu)
        sc = [empty_f32((M, Tp), gpu) for _ in range(4)]
        eg.engram_gateconv_fwd(*args, wh, wv, cw, Y, vh, *sc)
        return [Y, vh] + sc

    ref = fwd(T)
    torch.cuda.synchronize()
    sizes = sorted(set(range(1, 10)) | {15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 127, 128, 129, 255, 257,
                                        T // 3, T // 2, T - 4, T - 1})
    bad = []
    for Tp in sizes:
        got = fwd(Tp)
        torch.cuda.synchronize()
        if not all(_same(g, r[:, :Tp]) for g, r in zip(got, ref)):
            bad.append(Tp)
    assert not bad, f"GateConv forward prefixes differ at T' = {bad}"
