"""engram_gate_bwd_noalloc (no workspace; the library's own per-GPU partial
rows) against engram_gate_bwd (caller's workspace), called through the C ABI:
three calls in a row, each compared bit for bit with the workspace backward on
the same inputs and saved state, and the last also against the oracle.  The
first, N = 8128, fills 127 of the array's 128 partial rows (the most any
accepted N uses: 8128 / 64 rows, since 256 does not divide it); the second,
N = 8192, uses only 64 of them and the third, N = 1088, only 17, so stale
partial rows left by an earlier call would show."""
from __future__ import annotations

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def _noalloc(eg, d, saved, n):
    import torch
    from gpu_util import poison
    x, kv = d["x"], d["kv"]
    gx, gkv = poison(torch.empty_like(x)), poison(torch.empty_like(kv))
    gw = poison(torch.empty((4, 5120), dtype=torch.float32, device=x.device))
    st = eg.lib.engram_gate_bwd_noalloc(x.data_ptr(), kv.data_ptr(), d["weight"].data_ptr(), saved.data_ptr(),
                                        d["grad_out"].data_ptr(), gx.data_ptr(), gkv.data_ptr(), gw.data_ptr(), n,
                                        torch.cuda.current_stream(x.device).cuda_stream)
    assert st == eg.OK, eg.lib.engram_status_string(st)
    return gx, gkv, gw


def test_noalloc_backward_matches_workspace_backward(gpu):
    import torch
    import memory_bound_engram_amd as eg
    from gpu_util import dev_inputs, f32, run_bwd, run_fwd, u16
    from parity import check_bwd
    for n, seed, p, edge in ((8128, 7, 0.5, True), (8192, 0, 0.3, True), (1088, 5, 0.9, False)):
        print(f"noalloc call: N={n} seed={seed} mask p={p} edge rows={edge}", flush=True)
        inp = synth.host_inputs(n, seed=seed, p=p, grad=True, edge=edge)
        d = dev_inputs(inp, gpu)
        _, saved = run_fwd(d)
        ref = run_bwd(d, saved)
        got = _noalloc(eg, d, saved, n)
        torch.cuda.synchronize()
        for a, b in zip(ref, got):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    st = check_bwd(inp, f32(saved), u16(got[0]), u16(got[1]), f32(got[2]), threads=16)
    print(st)


def test_noalloc_rejects_sizes_beyond_its_array(gpu):
    import torch
    import memory_bound_engram_amd as eg
    x = torch.empty((64, 4, 5120), dtype=torch.bfloat16, device=gpu)
    p = x.data_ptr()
    # rejected on the host before any device access (the pointers are never used)
    assert eg.lib.engram_gate_bwd_noalloc(p, p, p, p, p, p, p, p, 8256, None) == eg.ERR_N_RANGE
    assert eg.lib.engram_gate_bwd_noalloc(p, p, p, p, p, p, p, p, 100, None) == eg.ERR_N_MULT64
    assert eg.lib.engram_gate_bwd_noalloc(p, p, p, p, p, p, p, p, 0, None) == eg.ERR_N_RANGE
    with pytest.raises(eg.EngramError):
        eg.engram_gate_bwd_noalloc(x, x, x, x, x, x, x, x, N=1 << 14)
