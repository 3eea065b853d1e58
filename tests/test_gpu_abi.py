"""C-ABI behaviour on the GPU: error returns leave outputs untouched, inputs
may alias each other, and the device generator matches the host generator."""
from __future__ import annotations

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


def test_rejected_calls_do_not_touch_outputs(gpu):
    import torch
    import memory_bound_engram_amd as eg
    from gpu_util import alloc_bwd, dev_inputs, poison
    inp = synth.host_inputs(100, seed=1, p=0.9, grad=True)
    d = dev_inputs(inp, gpu)
    gx, gkv, gw, ws = alloc_bwd(d["x"], d["kv"], 100)  # sized for N = 100: the library's own check fires
    saved = torch.zeros((100, 4, 4), dtype=torch.float32, device=gpu)
    with pytest.raises(eg.EngramError) as e:
        eg.engram_gate_bwd(d["x"], d["kv"], d["weight"], saved, d["grad_out"], gx, gkv, gw, ws, 100)
    assert e.value.status == eg.ERR_N_MULT64
    torch.cuda.synchronize()
    assert (gx.view(torch.int16) == -1).all()
    out = poison(torch.empty_like(d["x"]))
    with pytest.raises(eg.EngramError) as e:
        eg.engram_gate_fwd(d["x"], d["kv"], d["weight"], d["mask"], d["x"], saved, 100)
    assert e.value.status == eg.ERR_OVERLAP


def test_grad_out_may_alias_x(gpu):
    import torch
    import oracle
    from gpu_util import f32, run_bwd, to_dev, u16, dev_inputs
    from parity import check_bwd
    inp = synth.host_inputs(64, seed=2, p=0.9)
    inp["grad_out"] = inp["x"]
    d = dev_inputs({k: v for k, v in inp.items() if k != "grad_out"}, gpu)
    d["grad_out"] = d["x"]
    _, saved_ref = oracle.fwd_bf16(inp["x"], inp["kv"], inp["weight"], inp["mask"])
    gx, gkv, gw = run_bwd(d, to_dev(saved_ref, gpu))
    torch.cuda.synchronize()
    check_bwd(inp, saved_ref, u16(gx), u16(gkv), f32(gw))


@pytest.mark.parametrize("count,offset", [(1, 0), (7, 3), (4097, 12345), (1 << 20, 1 << 33)])
def test_device_generator_matches_host(gpu, count, offset):
    import torch
    from gpu_util import u16
    t = torch.empty(count + 8, dtype=torch.bfloat16, device=gpu)[:count]
    synth.dev_normal_bf16(t, 9, synth.ID_KV, offset)
    assert np.array_equal(u16(t), synth.normal_bf16(count, 9, synth.ID_KV, offset))
    m = torch.empty(count, dtype=torch.uint8, device=gpu)
    synth.dev_mask(m, 9, 0.3, offset)
    assert np.array_equal(m.cpu().numpy(), synth.mask(count, 9, 0.3, offset))
