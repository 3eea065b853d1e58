"""Forward parity: libengram on the GPU vs the fp64 oracle on the same bytes."""
from __future__ import annotations

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _run_and_check(gpu, inp, **kw):
    import torch
    from gpu_util import dev_inputs, f32, run_fwd, u16
    from parity import check_fwd
    d = dev_inputs(inp, gpu)
    out, saved = run_fwd(d)
    torch.cuda.synchronize()
    st = check_fwd(inp, u16(out), f32(saved), **kw)
    return st, u16(out), f32(saved)


def test_fwd_tiny_n64_mask09(gpu):
    """N = 64 tokens, mask Bernoulli(0.9), seed 0 (the smallest workload)."""
    inp = synth.host_inputs(64, seed=0, p=0.9)
    st, _, _ = _run_and_check(gpu, inp)
    print(st)


@pytest.mark.parametrize("n", [1, 2, 3, 7, 130, 333, 1000])
def test_fwd_ragged_sizes(gpu, n):
    """Sizes below, around and above the persistent grid; half the tokens masked."""
    inp = synth.host_inputs(n, seed=100 + n, p=0.5)
    _run_and_check(gpu, inp)


def test_fwd_all_masked_and_none_masked(gpu):
    for p in (0.0, 1.0):
        inp = synth.host_inputs(96, seed=7, p=p)
        _run_and_check(gpu, inp)


def test_fwd_edge_rows(gpu):
    """eps-path, clamp-path and all-zero rows (the edge-row recipe), mask 0.3."""
    n = 512
    inp = synth.host_inputs(n, seed=0, p=0.3, edge=True)
    st, out, saved = _run_and_check(gpu, inp)
    # zero rows give dot == 0 exactly and gate 1/2 exactly (sgn(0) = 0)
    for i, r in enumerate(synth.zero_rows(n, 0)):
        t, s = divmod(int(r), 4)
        assert saved[t, s, 1] == 0.0
        assert saved[t, s, 0] == (0.5 if inp["mask"][t] else 0.0)


def test_fwd_subnormal_rows(gpu):
    """bf16 subnormal inputs where the forward adds or scales them, mask all
    ones: tokens 0-31 have subnormal X rows and a zero value row, so out must
    be X bit for bit (out = x + gate * 0); tokens 32-63 have zero X rows and a
    subnormal value row, so dot = 0, gate = 1/2 and out = bf16(v / 2).  A
    flush to zero of a subnormal operand or result in the forward breaks the
    one-ulp bar on out; both sides take the dot of the subnormal X rows far
    inside the clamp (rstd_X = eps^-1/2)."""
    from numerics import subnormal_bf16
    n = 256
    inp = synth.host_inputs(n, seed=8, p=1.0)
    x, kv = inp["x"], inp["kv"]
    x[0:32] = subnormal_bf16(x[0:32])
    kv[0:32, 4 * 5120:] = 0
    x[32:64] = 0
    kv[32:64, 4 * 5120:] = subnormal_bf16(kv[32:64, 4 * 5120:])
    st, out, saved = _run_and_check(gpu, inp)
    assert np.array_equal(out[0:32], x[0:32]), "subnormal X not carried to out"
    assert np.all(saved[32:64, :, 0] == 0.5) and np.all(saved[32:64, :, 1] == 0.0)
    v = inp["kv"][32:64, 4 * 5120:]
    half = ((v.astype(np.uint32) << 16).view(np.float32).astype(np.float64) * 0.5)
    import oracle
    want = oracle.round_bf16(np.broadcast_to(half[:, None, :], (32, 4, 5120)))
    assert np.array_equal(out[32:64], want), "v / 2 of a subnormal value row"
    print(st)


def test_fwd_n8192_mask09(gpu):
    """N = 8192, mask Bernoulli(0.9): every element compared."""
    inp = synth.host_inputs(8192, seed=0, p=0.9)
    st, _, _ = _run_and_check(gpu, inp, threads=16)
    print(st)


def test_fwd_repeatable_bitwise(gpu):
    import torch
    from gpu_util import dev_inputs, run_fwd
    inp = synth.host_inputs(777, seed=3, p=0.8)
    d = dev_inputs(inp, gpu)
    o1, s1 = run_fwd(d)
    o2, s2 = run_fwd(d)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))


def test_fwd_side_stream(gpu):
    import torch
    from gpu_util import dev_inputs, f32, run_fwd, u16
    from parity import check_fwd
    inp = synth.host_inputs(200, seed=4, p=0.9)
    d = dev_inputs(inp, gpu)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, saved = run_fwd(d, stream=s)
    s.synchronize()
    check_fwd(inp, u16(out), f32(saved))


def test_fwd_one_million_tokens_sampled(gpu):
    """N = 1,048,512 in a single launch (~140 GB resident), device-generated
    inputs; sampled tokens compared with the oracle, whole-batch properties
    checked on the device; then N - 37 over the same inputs reproduces those
    tokens bit for bit and writes nothing past its end."""
    import torch
    import oracle
    from gpu_util import u16, f32
    import memory_bound_engram_amd as eg
    from parity import check_fwd
    n, seed, p = 1_048_512, 0, 0.9
    free, total = torch.cuda.mem_get_info(gpu)
    need = n * (40960 * 3 + 51200 + 64 * 2 + 1) + (1 << 30)  # inputs, two sets of outputs
    if free < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB of device memory, {free / 2**30:.0f} free")
    x = torch.empty((n, 4, 5120), dtype=torch.bfloat16, device=gpu)
    kv = torch.empty((n, 25600), dtype=torch.bfloat16, device=gpu)
    m = torch.empty(n, dtype=torch.uint8, device=gpu)
    synth.dev_normal_bf16(x, seed, synth.ID_X)
    synth.dev_normal_bf16(kv, seed, synth.ID_KV)
    synth.dev_mask(m, seed, p)
    w = torch.from_numpy(synth.normal_f32(4 * 5120, seed, synth.ID_W, 1.0, 0.1).reshape(4, 5120)).to(gpu)
    out = torch.empty_like(x)
    saved = torch.empty((n, 4, 4), dtype=torch.float32, device=gpu)
    out[-64:].view(torch.int16).fill_(-1)  # the tail must be overwritten
    eg.engram_gate_fwd(x, kv, w, m, out, saved, n)
    torch.cuda.synchronize()
    # sampled tokens: first, last, and random ones, regenerated on the host
    rng = np.random.default_rng(1)
    toks = np.unique(np.concatenate([np.arange(8), np.arange(n - 8, n), rng.integers(0, n, 48)]))
    for t in toks:
        inp = synth.host_inputs(n, seed=seed, p=p, t0=int(t), nt=1)
        assert np.array_equal(u16(x[t:t + 1]), inp["x"]), "device generator differs from host"
        check_fwd(inp, u16(out[t:t + 1]), f32(saved[t:t + 1]))
    # whole-batch properties, in chunks
    step = 16384
    for t0 in range(0, n, step):
        sl = slice(t0, min(n, t0 + step))
        on = m[sl] != 0
        sv = saved[sl]
        assert torch.isfinite(sv).all()
        assert (sv[~on][:, :, 0] == 0).all()
        g = sv[on][:, :, 0]
        assert ((g > 0) & (g <= 1)).all()  # sigmoid of a large z rounds to 1.0f
        ob = out[sl].view(torch.int16)
        xb = x[sl].view(torch.int16)
        assert torch.equal(ob[~on], xb[~on])
        assert torch.isfinite(out[sl][on].float()).all()
    # a ragged size over the same inputs (the grid-stride tail at this scale):
    # the first n2 tokens bit for bit as above, nothing past n2 written
    n2 = n - 37
    out2 = torch.empty_like(x)
    saved2 = torch.empty_like(saved)
    out2[n2 - 64:].view(torch.int16).fill_(-1)
    saved2[n2 - 64:].view(torch.int32).fill_(-1)
    eg.engram_gate_fwd(x, kv, w, m, out2, saved2, n2)
    torch.cuda.synchronize()
    for t0 in range(0, n2, step):
        sl = slice(t0, min(n2, t0 + step))
        assert torch.equal(out2[sl].view(torch.int16), out[sl].view(torch.int16)), f"out differs near token {t0}"
        assert torch.equal(saved2[sl].view(torch.int32), saved[sl].view(torch.int32)), f"saved differs near token {t0}"
    assert (out2[n2:].view(torch.int16) == -1).all() and (saved2[n2:].view(torch.int32) == -1).all()
    del x, kv, out, saved, out2, saved2
    torch.cuda.empty_cache()
