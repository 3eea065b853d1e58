"""Backward parity: libengram on the GPU vs the fp64 oracle.

As in the tile-kernels backward test, the backward is checked on the
reference forward's saved intermediates: the oracle's fp32 saved is uploaded
and both sides consume it.  The device-only chain (device forward -> device
backward) is checked norm-wise against the oracle chain."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth

pytestmark = pytest.mark.gpu


def _bwd_case(gpu, inp, threads=8):
    import torch
    from gpu_util import dev_inputs, f32, run_bwd, to_dev, u16
    from parity import check_bwd
    _, saved_ref = oracle.fwd_bf16(inp["x"], inp["kv"], inp["weight"], inp["mask"], threads=threads)
    d = dev_inputs(inp, gpu)
    gx, gkv, gw = run_bwd(d, to_dev(saved_ref, gpu))
    torch.cuda.synchronize()
    st = check_bwd(inp, saved_ref, u16(gx), u16(gkv), f32(gw), threads=threads)
    return st, saved_ref, u16(gx), u16(gkv), f32(gw)


def test_bwd_n64(gpu):
    inp = synth.host_inputs(64, seed=0, p=0.9, grad=True)
    st, *_ = _bwd_case(gpu, inp)
    print(st)


@pytest.mark.parametrize("n", [128, 192, 640, 1088])
def test_bwd_block_counts(gpu, n):
    """2, 3, 10 and 17 partial rows: uneven chunks in the grad_weight reduction."""
    inp = synth.host_inputs(n, seed=n, p=0.7, grad=True)
    _bwd_case(gpu, inp)


@pytest.mark.parametrize("n", [4160, 4224, 4352, 4608, 6144, 7936, 8128])
def test_bwd_row_partitions_above_4096(gpu, n):
    """The backward's other token partitions above N = 4096: 64 rows of N/256
    steps when 256 divides N (4352, 4608, 6144, 7936: 17, 18, 24 and 31 steps),
    and N/64 rows walked in two rounds of workgroups when it does not (4160,
    4224: 65 and 66 rows; 8128: 127 rows, the most the workspace holds)."""
    inp = synth.host_inputs(n, seed=n, p=0.7, grad=True)
    st, *_ = _bwd_case(gpu, inp, threads=16)
    print(st)


def test_bwd_subnormal_rows(gpu):
    """bf16 subnormal inputs where the backward multiplies them: tokens 0-31
    have subnormal grad_out rows, tokens 32-63 subnormal value rows, tokens
    64-95 both; the rest are normal.  The oracle is exact on them, so a flush
    to zero anywhere in dg or the outputs fails the elementwise bars (a CPU
    test checks that a planted flush is caught)."""
    from gpu_util import dev_inputs, f32, run_bwd, to_dev, u16
    from numerics import subnormal_rows_case
    from parity import check_bwd
    import torch
    inp = subnormal_rows_case()
    _, saved_ref = oracle.fwd_bf16(inp["x"], inp["kv"], inp["weight"], inp["mask"], threads=8)
    d = dev_inputs(inp, gpu)
    gx, gkv, gw = run_bwd(d, to_dev(saved_ref, gpu))
    torch.cuda.synchronize()
    st = check_bwd(inp, saved_ref, u16(gx), u16(gkv), f32(gw), threads=8)
    print(st)


def test_fwd_bwd_n4096(gpu):
    """N = 4096, mask 0.9, grad_out N(0,1): forward parity, backward parity on
    the oracle's saved, and the device-only chain norm-wise."""
    import torch
    from gpu_util import dev_inputs, f32, run_bwd, run_fwd, u16
    from parity import check_bwd_end_to_end, check_fwd
    inp = synth.host_inputs(4096, seed=0, p=0.9, grad=True)
    st_b, saved_ref, *_ = _bwd_case(gpu, inp, threads=16)
    d = dev_inputs(inp, gpu)
    out, saved = run_fwd(d)
    gx, gkv, gw = run_bwd(d, saved)
    torch.cuda.synchronize()
    fwd_ref = oracle.fwd_bf16(inp["x"], inp["kv"], inp["weight"], inp["mask"], threads=16, extras=True)
    st_f = check_fwd(inp, u16(out), f32(saved), ref=fwd_ref)
    st_e = check_bwd_end_to_end(inp, f32(saved), u16(gx), u16(gkv), f32(gw), fwd_ref, threads=16)
    print(st_f, st_b, st_e)


def test_bwd_n8192_edge_rows(gpu):
    """N = 8192 (the backward maximum), mask 0.3, eps/clamp/zero rows."""
    from numerics import bf16_to_f64
    n = 8192
    inp = synth.host_inputs(n, seed=0, p=0.3, grad=True, edge=True)
    st, saved_ref, dx, dkv, dw = _bwd_case(gpu, inp, threads=16)
    print(st)
    off = inp["mask"] == 0
    # masked tokens: dx = G bit for bit, key and value gradients zero
    assert np.array_equal(dx[off], inp["grad_out"][off])
    assert np.all(bf16_to_f64(dkv[off]) == 0.0)
    # clamp rows (|dot| < 1e-6): dx = G and dk = 0 on that stream
    dots = saved_ref[:, :, 1]
    t_idx, s_idx = np.nonzero((np.abs(dots) < np.float32(1e-6)) & ~off[:, None])
    assert t_idx.size > 100
    for t, s in zip(t_idx[:64], s_idx[:64]):
        assert np.array_equal(dx[t, s], inp["grad_out"][t, s])
        assert np.all(bf16_to_f64(dkv[t, s * 5120:(s + 1) * 5120]) == 0.0)


def test_bwd_all_masked(gpu):
    """Every token masked: the backward reads only grad_out and saved, and
    writes grad_x = grad_out bit for bit, grad_kv = +0 and grad_weight = 0."""
    import torch
    from gpu_util import dev_inputs, f32, run_bwd, run_fwd, u16
    n = 256
    inp = synth.host_inputs(n, seed=3, p=0.0, grad=True)
    assert not inp["mask"].any()
    d = dev_inputs(inp, gpu)
    out, saved = run_fwd(d)
    gx, gkv, gw = run_bwd(d, saved)
    torch.cuda.synchronize()
    assert np.array_equal(u16(out), inp["x"])
    assert np.all(f32(saved)[:, :, 0] == 0.0)
    assert np.array_equal(u16(gx), inp["grad_out"])
    assert not u16(gkv).any()
    assert not f32(gw).any()


def _keys_scaled(kv, k):
    """The four key blocks of bf16 KV rows times 2^k, exactly; the value stays."""
    out = kv.copy()
    f = (kv[:, :4 * 5120].astype(np.uint32) << 16).view(np.float32)
    g = f * np.float32(2.0 ** k)
    out[:, :4 * 5120] = (g.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((out[:, :4 * 5120].astype(np.uint32) << 16).view(np.float32), g), "scale not exact"
    return out


def test_bwd_all_clamp_n8192(gpu):
    """N = 8192 (64 rows of 128 tokens), every key times 2^-64: its squares
    fall far below eps, so rstd_key ~ eps^-1/2 leaves the normalised key ~1e-9
    and |dot| < 1e-6 on every stream of every token.  Every unmasked token
    takes the clamp path (delta = 0): grad_x = G bit for bit, grad_key = +0,
    grad_weight = 0, and grad_value = sum_s gate_s G_s alone, against the
    oracle on its saved state and on the device's own."""
    import torch
    from gpu_util import dev_inputs, f32, run_bwd, run_fwd, u16
    from numerics import bf16_to_f64
    from parity import check_bwd_end_to_end, check_fwd
    n = 8192
    inp = synth.host_inputs(n, seed=5, p=0.9, grad=True)
    inp["kv"] = _keys_scaled(inp["kv"], -64)
    st_b, saved_ref, *_ = _bwd_case(gpu, inp, threads=16)
    assert np.all(np.abs(saved_ref[:, :, 1]) < np.float32(1e-6))
    d = dev_inputs(inp, gpu)
    out, saved = run_fwd(d)
    gx, gkv, gw = run_bwd(d, saved)
    torch.cuda.synchronize()
    sv = f32(saved)
    assert np.all(np.abs(sv[:, :, 1]) < np.float32(1e-6)), "a stream left the clamp path"
    assert np.array_equal(u16(gx), inp["grad_out"]), "grad_x is not G"
    assert not u16(gkv)[:, :4 * 5120].any(), "grad_key is not +0"
    assert not f32(gw).any(), "grad_weight is not 0"
    on = inp["mask"] != 0
    assert np.any(bf16_to_f64(u16(gkv)[on, 4 * 5120:]) != 0.0)
    fwd_ref = oracle.fwd_bf16(inp["x"], inp["kv"], inp["weight"], inp["mask"], threads=16, extras=True)
    st_f = check_fwd(inp, u16(out), sv, ref=fwd_ref)
    st_e = check_bwd_end_to_end(inp, sv, u16(gx), u16(gkv), f32(gw), fwd_ref, threads=16)
    print(st_f, st_b, st_e)


def test_bwd_all_masked_n8192(gpu):
    """Every token masked at N = 8192 (64 rows of 128 tokens): grad_x = G bit
    for bit, grad_kv = +0, grad_weight = 0."""
    import torch
    from gpu_util import dev_inputs, f32, run_bwd, run_fwd, u16
    n = 8192
    inp = synth.host_inputs(n, seed=6, p=0.0, grad=True)
    assert not inp["mask"].any()
    d = dev_inputs(inp, gpu)
    out, saved = run_fwd(d)
    gx, gkv, gw = run_bwd(d, saved)
    torch.cuda.synchronize()
    assert np.array_equal(u16(out), inp["x"])
    assert np.all(f32(saved)[:, :, 0] == 0.0)
    assert np.array_equal(u16(gx), inp["grad_out"])
    assert not u16(gkv).any()
    assert not f32(gw).any()


def test_fwd_bwd_repeated_1000_bitwise(gpu):
    """N = 8192 with the edge-row recipe, mask 0.3: 1000 forward+backward
    launches back to back on one stream; the last results equal the first
    bit for bit (no state carried through the workspace)."""
    import torch
    import memory_bound_engram_amd as eg
    from gpu_util import alloc_bwd, dev_inputs, poison
    n = 8192
    inp = synth.host_inputs(n, seed=0, p=0.3, grad=True, edge=True)
    d = dev_inputs(inp, gpu)
    x, kv, w, m, g = d["x"], d["kv"], d["weight"], d["mask"], d["grad_out"]

    def one(out, saved, gx, gkv, gw, ws):
        eg.engram_gate_fwd(x, kv, w, m, out, saved, n)
        eg.engram_gate_bwd(x, kv, w, saved, g, gx, gkv, gw, ws, n)

    first = [poison(torch.empty_like(x)), poison(torch.empty((n, 4, 4), dtype=torch.float32, device=gpu)),
             *alloc_bwd(x, kv, n)]
    one(*first)
    again = [poison(torch.empty_like(x)), poison(torch.empty((n, 4, 4), dtype=torch.float32, device=gpu)),
             *alloc_bwd(x, kv, n)]
    for _ in range(1000):
        one(*again)
    torch.cuda.synchronize()
    for a, b in zip(first[:5], again[:5]):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_config4_fwd_bwd_1000_launches_vs_oracle(gpu):
    """The edge-row workload as a whole: N = 8192 (the backward maximum),
    mask Bernoulli(0.3), 5% of rows with X or a key scaled by 1e-12 (eps
    path), 10% with keys inside the clamp band, all-zero rows; 1000 forward +
    backward launches back to back on one stream, then the last launch's
    results against the oracle on the same input bytes:
      - the device forward, every element (out, saved);
      - the device backward on the device's own saved, elementwise, with the
        oracle consuming that same saved;
      - the device chain against the oracle chain (oracle forward, then
        oracle backward), norm-wise;
      - masked and clamp-path rows exactly (grad_x = grad_out bit for bit,
        grad_key = 0)."""
    import torch
    import memory_bound_engram_amd as eg
    from gpu_util import alloc_bwd, dev_inputs, f32, poison, u16
    from numerics import bf16_to_f64
    from parity import check_bwd, check_bwd_end_to_end, check_fwd
    n = 8192
    inp = synth.host_inputs(n, seed=0, p=0.3, grad=True, edge=True)
    counts = inp["edge_counts"]
    print("edge rows:", counts, flush=True)
    d = dev_inputs(inp, gpu)
    x, kv, w, m, g = d["x"], d["kv"], d["weight"], d["mask"], d["grad_out"]
    out = poison(torch.empty_like(x))
    saved = poison(torch.empty((n, 4, 4), dtype=torch.float32, device=gpu))
    gx, gkv, gw, ws = alloc_bwd(x, kv, n)
    for _ in range(1000):
        eg.engram_gate_fwd(x, kv, w, m, out, saved, n)
        eg.engram_gate_bwd(x, kv, w, saved, g, gx, gkv, gw, ws, n)
    torch.cuda.synchronize()
    out_h, saved_h = u16(out), f32(saved)
    dx, dkv, dw = u16(gx), u16(gkv), f32(gw)
    fwd_ref = oracle.fwd_bf16(inp["x"], inp["kv"], inp["weight"], inp["mask"], threads=16, extras=True)
    st_f = check_fwd(inp, out_h, saved_h, ref=fwd_ref)
    st_b = check_bwd(inp, saved_h, dx, dkv, dw, threads=16)
    st_e = check_bwd_end_to_end(inp, saved_h, dx, dkv, dw, fwd_ref, threads=16)
    print(st_f, st_b, st_e)
    off = inp["mask"] == 0
    assert np.array_equal(dx[off], inp["grad_out"][off])
    assert np.all(bf16_to_f64(dkv[off]) == 0.0)
    dots = saved_h[:, :, 1]
    clamp = np.abs(dots) < np.float32(1e-6)
    assert 0.08 < clamp.mean() < 0.12          # the workload puts 10% of the dots inside the clamp
    t_idx, s_idx = np.nonzero(clamp & ~off[:, None])
    assert t_idx.size > 100
    for t, s in zip(t_idx, s_idx):
        assert np.array_equal(dx[t, s], inp["grad_out"][t, s])
        assert np.all(bf16_to_f64(dkv[t, s * 5120:(s + 1) * 5120]) == 0.0)
