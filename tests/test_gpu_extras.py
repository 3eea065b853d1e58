"""The steps either side of the hot path and graph capture (GPU):

- fused weight = wh * we, bit-exact against the oracle (the tile-kernels
  fused-weight test requires exact equality);
- the inference forward (saved = NULL) writes the same bits as the saving one
  (the tile-kernels forward test requires this of save_for_backward=False);
- the backward with the product rule writes grad_wh = grad_weight * we and
  grad_we = grad_weight * wh, checked against the oracle's product rule;
- forward + backward captured in a HIP graph replay to the eager results.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _norm_weights(seed):
    wh = synth.normal_bf16(4 * 5120, seed, 21).reshape(4, 5120)
    we = synth.normal_bf16(4 * 5120, seed, 22).reshape(4, 5120)
    return wh, we


def test_fused_weight_bit_exact(gpu):
    import torch
    import memory_bound_engram_amd as eg
    from gpu_util import poison, to_dev
    wh, we = _norm_weights(5)
    w = poison(torch.empty((4, 5120), dtype=torch.float32, device=gpu))
    eg.engram_fused_weight(to_dev(wh, gpu), to_dev(we, gpu), w)
    torch.cuda.synchronize()
    ref = oracle.fused_weight(wh, we)
    assert np.array_equal(w.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_fwd_without_saved_is_bit_identical(gpu):
    import torch
    import memory_bound_engram_amd as eg
    from gpu_util import dev_inputs, poison, run_fwd, u16
    inp = synth.host_inputs(333, seed=8, p=0.7)
    d = dev_inputs(inp, gpu)
    out_s, _ = run_fwd(d)
    out_n = poison(torch.empty_like(d["x"]))
    eg.engram_gate_fwd(d["x"], d["kv"], d["weight"], d["mask"], out_n, None, 333)
    torch.cuda.synchronize()
    assert np.array_equal(u16(out_s), u16(out_n))


def test_bwd_with_norm_weights(gpu):
    import torch
    import memory_bound_engram_amd as eg
    from gpu_util import alloc_bwd, dev_inputs, poison, to_dev, u16
    n = 1088
    wh, we = _norm_weights(6)
    inp = synth.host_inputs(n, seed=6, p=0.8, grad=True)
    inp["weight"] = oracle.fused_weight(wh, we)
    _, saved_ref = oracle.fwd_bf16(inp["x"], inp["kv"], inp["weight"], inp["mask"], threads=8)
    d = dev_inputs(inp, gpu)
    sv = to_dev(saved_ref, gpu)
    dwh, dwe = to_dev(wh, gpu), to_dev(we, gpu)
    a = alloc_bwd(d["x"], d["kv"], n)
    eg.engram_gate_bwd(d["x"], d["kv"], d["weight"], sv, d["grad_out"], a[0], a[1], a[2], a[3], n)
    b = alloc_bwd(d["x"], d["kv"], n)
    gwh = poison(torch.empty((4, 5120), dtype=torch.float32, device=gpu))
    gwe = poison(torch.empty((4, 5120), dtype=torch.float32, device=gpu))
    eg.engram_gate_bwd_with_norm_weights(d["x"], d["kv"], d["weight"], sv, d["grad_out"], b[0], b[1], b[2],
                                         dwh, dwe, gwh, gwe, b[3], n)
    torch.cuda.synchronize()
    # the same kernels: grad_x, grad_kv, grad_weight are bit-identical to the plain call
    for p, q in zip(a[:3], b[:3]):
        assert torch.equal(p.view(torch.uint8), q.view(torch.uint8))
    # the product rule is one fp32 multiply of the device's own grad_weight
    dw_dev = b[2].cpu().numpy()
    whf = (wh.astype(np.uint32) << 16).view(np.float32)
    wef = (we.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(gwh.cpu().numpy(), dw_dev * wef)
    assert np.array_equal(gwe.cpu().numpy(), dw_dev * whf)
    # and agrees with the oracle's product rule within grad_weight's bar
    ref = oracle.bwd_bf16(inp["x"], inp["kv"], inp["weight"], saved_ref, inp["grad_out"], threads=8, extras=True)
    dw64, mdw = ref[5], ref[8]
    rwh, rwe = oracle.weight_grads(dw64, wh, we)
    tol_dw = 1e-3 * np.abs(dw64) + 2.0 ** -17 * mdw
    for got, want, fac in ((gwh, rwh, np.abs(wef)), (gwe, rwe, np.abs(whf))):
        diff = np.abs(got.cpu().numpy().astype(np.float64) - want)
        assert np.all(diff <= fac * tol_dw + 2.0 ** -23 * np.abs(want)), float(diff.max())


def test_graph_capture_replays_match_eager(gpu):
    """forward + backward captured once, replayed four times with eager work
    and synchronisations in between; every replay equals the eager result."""
    import torch
    import memory_bound_engram_amd as eg
    from gpu_util import alloc_bwd, dev_inputs, poison
    n = 1024
    inp = synth.host_inputs(n, seed=9, p=0.8, grad=True)
    d = dev_inputs(inp, gpu)
    x, kv, w, m, g = d["x"], d["kv"], d["weight"], d["mask"], d["grad_out"]
    out = torch.empty_like(x)
    saved = torch.empty((n, 4, 4), dtype=torch.float32, device=gpu)
    gx, gkv, gw, ws = alloc_bwd(x, kv, n)

    def step():
        eg.engram_gate_fwd(x, kv, w, m, out, saved, n)
        eg.engram_gate_bwd(x, kv, w, saved, g, gx, gkv, gw, ws, n)

    step()  # eager reference (also warms the library's per-device caches)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, saved, gx, gkv, gw)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        for t in (out, saved, gx, gkv, gw, ws):
            poison(t)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, (out, saved, gx, gkv, gw)):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {r} differs"
        torch.ones(1 << 20, device=gpu).cumsum(0)  # unrelated eager work between replays


def test_graph_replays_config4_loop_1000(gpu):
    """The 1000-launch loop of N = 8192 with the edge-row recipe and mask 0.3,
    replayed from a HIP graph: one captured forward + backward, replayed 1000
    times on one stream; outputs (poisoned before the loop) equal the eager
    result bit for bit, and a spot check every 250 replays does too."""
    import torch
    import memory_bound_engram_amd as eg
    from gpu_util import alloc_bwd, dev_inputs, poison
    n = 8192
    inp = synth.host_inputs(n, seed=0, p=0.3, grad=True, edge=True)
    d = dev_inputs(inp, gpu)
    x, kv, w, m, g = d["x"], d["kv"], d["weight"], d["mask"], d["grad_out"]
    out = torch.empty_like(x)
    saved = torch.empty((n, 4, 4), dtype=torch.float32, device=gpu)
    gx, gkv, gw, ws = alloc_bwd(x, kv, n)

    def step():
        eg.engram_gate_fwd(x, kv, w, m, out, saved, n)
        eg.engram_gate_bwd(x, kv, w, saved, g, gx, gkv, gw, ws, n)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, saved, gx, gkv, gw)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step()
    torch.cuda.synchronize()
    for t in (out, saved, gx, gkv, gw, ws):
        poison(t)
    torch.cuda.synchronize()
    for i in range(1000):
        graph.replay()
        if i % 250 == 249:
            torch.cuda.synchronize()
            for a, b in zip(ref, (out, saved, gx, gkv, gw)):
                assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {i} differs"
    torch.cuda.synchronize()
