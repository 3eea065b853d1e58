"""The forward's paced path (calls longer than 16384 tokens): one workgroup
per CU walking the tokens in epochs, with a bounded-wait barrier between
epochs.  The barrier only paces, so the paced call must give the unpaced
kernel's results bit for bit: every test compares a long call with the same
tokens run as calls of at most 16384 tokens (the unpaced path), on ragged
sizes whose last epoch is partly empty, nothing written past N; sampled
tokens are also compared with the oracle.  The barrier's counters live in a
small device array that the calls deal round robin and reset themselves;
repeated calls, calls on two streams at once and graph replays must all keep
both the results and the speed (a barrier that never releases would wait out
its bound every epoch, ~1.4 ms more on a 65536-token call)."""
from __future__ import annotations

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

PACED_MIN = 16384  # calls above this many tokens take the paced path
SEED, P = 5, 0.9


def _inputs(torch, gpu, n, pad=0):
    x = torch.empty((n + pad, 4, 5120), dtype=torch.bfloat16, device=gpu)
    kv = torch.empty((n + pad, 25600), dtype=torch.bfloat16, device=gpu)
    m = torch.empty(n + pad, dtype=torch.uint8, device=gpu)
    synth.dev_normal_bf16(x, SEED, synth.ID_X)
    synth.dev_normal_bf16(kv, SEED, synth.ID_KV)
    synth.dev_mask(m, SEED, P)
    w = torch.from_numpy(synth.normal_f32(4 * 5120, SEED, synth.ID_W, 1.0, 0.1).reshape(4, 5120)).to(gpu)
    return x, kv, w, m


def _chunked(eg, x, kv, w, m, out, saved, n, chunk=PACED_MIN):
    for t0 in range(0, n, chunk):
        c = min(chunk, n - t0)
        eg.engram_gate_fwd(x[t0:t0 + c], kv[t0:t0 + c], w, m[t0:t0 + c], out[t0:t0 + c],
                           None if saved is None else saved[t0:t0 + c], c)


@pytest.mark.parametrize("n", [PACED_MIN + 1, 3 * 8192 + 5, 65536, 131_079])
def test_paced_equals_unpaced(gpu, n):
    import torch
    import memory_bound_engram_amd as eg
    from gpu_util import f32, u16
    from parity import check_fwd
    pad = 64
    x, kv, w, m = _inputs(torch, gpu, n, pad)
    ref_out = torch.empty_like(x)
    ref_saved = torch.empty((n + pad, 4, 4), dtype=torch.float32, device=gpu)
    _chunked(eg, x, kv, w, m, ref_out, ref_saved, n)
    out = torch.empty_like(x)
    saved = torch.empty_like(ref_saved)
    out.view(torch.int16).fill_(-1)
    saved.view(torch.int32).fill_(-1)
    eg.engram_gate_fwd(x, kv, w, m, out, saved, n)
    torch.cuda.synchronize()
    assert torch.equal(out[:n].view(torch.int16), ref_out[:n].view(torch.int16))
    assert torch.equal(saved[:n].view(torch.int32), ref_saved[:n].view(torch.int32))
    assert (out[n:].view(torch.int16) == -1).all(), "paced forward wrote past N (out)"
    assert (saved[n:].view(torch.int32) == -1).all(), "paced forward wrote past N (saved)"
    # the inference forward on the paced path: same out, nothing saved
    out2 = torch.empty_like(x)
    out2.view(torch.int16).fill_(-1)
    eg.engram_gate_fwd(x, kv, w, m, out2, None, n)
    torch.cuda.synchronize()
    assert torch.equal(out2[:n].view(torch.int16), ref_out[:n].view(torch.int16))
    assert (out2[n:].view(torch.int16) == -1).all()
    # sampled tokens (first, last, around epoch edges, random) against the oracle
    rng = np.random.default_rng(n)
    toks = np.unique(np.concatenate([[0, 1, 255, 256, 8191, 8192, n - 2, n - 1], rng.integers(0, n, 8)]))
    for t in toks[toks < n]:
        inp = synth.host_inputs(n + pad, seed=SEED, p=P, t0=int(t), nt=1)
        assert np.array_equal(u16(x[t:t + 1]), inp["x"]), "device generator differs from host"
        check_fwd(inp, u16(out[t:t + 1]), f32(saved[t:t + 1]))


def _time_ms(torch, fn, reps):
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def test_paced_repeated_calls_keep_results_and_speed(gpu):
    """40 calls in a row (the 16 counter slots dealt 2.5 times over): each
    bit-identical to the first, and per call no slower than 1.5x the same
    tokens run unpaced."""
    import torch
    import memory_bound_engram_amd as eg
    n = 65536
    x, kv, w, m = _inputs(torch, gpu, n)
    out = torch.empty_like(x)
    saved = torch.empty((n, 4, 4), dtype=torch.float32, device=gpu)
    eg.engram_gate_fwd(x, kv, w, m, out, saved, n)
    torch.cuda.synchronize()
    ref_out, ref_saved = out.clone(), saved.clone()
    for i in range(40):
        out.view(torch.int16).fill_(-1)
        eg.engram_gate_fwd(x, kv, w, m, out, saved, n)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"call {i}"
        assert torch.equal(saved.view(torch.int32), ref_saved.view(torch.int32)), f"call {i}"
    paced = _time_ms(torch, lambda: eg.engram_gate_fwd(x, kv, w, m, out, saved, n), 20)
    unpaced = _time_ms(torch, lambda: _chunked(eg, x, kv, w, m, out, saved, n), 20)
    print(f"N={n}: paced {paced * 1e3:.1f} us, as 16384-token calls {unpaced * 1e3:.1f} us")
    assert paced < 1.5 * unpaced


def test_paced_two_streams_at_once(gpu):
    """Two paced calls enqueued on two streams without a wait between them
    (different inputs, different counter slots): both equal their results
    run alone."""
    import torch
    import memory_bound_engram_amd as eg
    n = 40_000
    a = _inputs(torch, gpu, n)
    b = [t.clone() for t in a]
    b[0].mul_(-0.5)  # different data on the second stream
    outs, refs = [], []
    for args in (a, b):
        o = torch.empty_like(args[0])
        sv = torch.empty((n, 4, 4), dtype=torch.float32, device=gpu)
        eg.engram_gate_fwd(*args, o, sv, n)
        torch.cuda.synchronize()
        refs.append((o.clone(), sv.clone()))
        o.view(torch.int16).fill_(-1)
        outs.append((o, sv))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for s, args, (o, sv) in zip(streams, (a, b), outs):
            with torch.cuda.stream(s):
                eg.engram_gate_fwd(*args, o, sv, n)
        torch.cuda.synchronize()
        for (o, sv), (ro, rs) in zip(outs, refs):
            assert torch.equal(o.view(torch.int16), ro.view(torch.int16)), f"rep {rep}"
            assert torch.equal(sv.view(torch.int32), rs.view(torch.int32)), f"rep {rep}"
            o.view(torch.int16).fill_(-1)
        torch.cuda.synchronize()


def test_paced_graph_replays(gpu):
    """A paced call captured in a graph (its counter slot fixed at capture)
    replayed five times with eager paced calls and other work in between:
    every replay bit-identical to the eager call, and as fast."""
    import torch
    import memory_bound_engram_amd as eg
    from gpu_util import poison
    n = 32768 + 5
    x, kv, w, m = _inputs(torch, gpu, n)
    out = torch.empty_like(x)
    saved = torch.empty((n, 4, 4), dtype=torch.float32, device=gpu)
    eg.engram_gate_fwd(x, kv, w, m, out, saved, n)
    torch.cuda.synchronize()
    ref = (out.clone(), saved.clone())
    other = torch.empty_like(out)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        eg.engram_gate_fwd(x, kv, w, m, out, saved, n)
    torch.cuda.synchronize()
    for r in range(5):
        poison(out)
        poison(saved)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref[0].view(torch.int16)), f"replay {r}"
        assert torch.equal(saved.view(torch.int32), ref[1].view(torch.int32)), f"replay {r}"
        eg.engram_gate_fwd(x, kv, w, m, other, None, n)  # eager paced call between replays
        torch.ones(1 << 20, device=gpu).cumsum(0)
    torch.cuda.synchronize()
    assert torch.equal(other.view(torch.int16), ref[0].view(torch.int16))
    replay = _time_ms(torch, graph.replay, 10)
    eager = _time_ms(torch, lambda: eg.engram_gate_fwd(x, kv, w, m, out, saved, n), 10)
    print(f"N={n}: graph replay {replay * 1e3:.1f} us, eager {eager * 1e3:.1f} us")
    assert replay < 1.5 * eager


def test_paced_results_do_not_depend_on_the_barrier(gpu, monkeypatch):
    """ENGRAM_PACE_WAIT_US=0: the first wait at the pacing barrier runs out at
    once and marks the call's slot abandoned, so every later wait returns at
    once (the kernel still counts through every barrier and resets its slot).
    The results stay bit-identical to the unpaced path, and a normally paced
    call right after still finds its slot clean (same results, no slower than
    1.5x the unpaced path)."""
    import torch
    import memory_bound_engram_amd as eg
    n = 3 * 8192 * 2 + 77
    x, kv, w, m = _inputs(torch, gpu, n)
    ref_out = torch.empty_like(x)
    ref_saved = torch.empty((n, 4, 4), dtype=torch.float32, device=gpu)
    _chunked(eg, x, kv, w, m, ref_out, ref_saved, n)
    out = torch.empty_like(x)
    saved = torch.empty_like(ref_saved)
    monkeypatch.setenv("ENGRAM_PACE_WAIT_US", "0")
    for i in range(20):  # more calls than counter slots
        out.view(torch.int16).fill_(-1)
        eg.engram_gate_fwd(x, kv, w, m, out, saved, n)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"unpaced call {i}"
        assert torch.equal(saved.view(torch.int32), ref_saved.view(torch.int32)), f"unpaced call {i}"
    monkeypatch.delenv("ENGRAM_PACE_WAIT_US")
    out.view(torch.int16).fill_(-1)
    eg.engram_gate_fwd(x, kv, w, m, out, saved, n)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16))
    paced = _time_ms(torch, lambda: eg.engram_gate_fwd(x, kv, w, m, out, saved, n), 20)
    unpaced = _time_ms(torch, lambda: _chunked(eg, x, kv, w, m, out, saved, n), 20)
    print(f"N={n}: paced {paced * 1e3:.1f} us after the no-wait calls, as 16384-token calls {unpaced * 1e3:.1f} us")
    assert paced < 1.5 * unpaced
