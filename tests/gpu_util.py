"""Device plumbing for the GPU tests: move numpy storage arrays to torch device
memory and back, and call libengram through its C ABI binding.  Outputs and
workspace are pre-filled with all-ones bytes (bf16/fp32 NaN) so that any
element a kernel fails to write shows up in the comparison."""
from __future__ import annotations

import numpy as np
import torch

import memory_bound_engram_amd as eg

D = 5120


def to_dev(a: np.ndarray, dev):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev)


def u16(t) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32(t) -> np.ndarray:
    return t.float().cpu().numpy()


def poison(t):
    t.view(torch.uint8).fill_(0xFF)
    return t


def dev_inputs(inp, dev):
    d = {k: to_dev(inp[k], dev) for k in ("x", "kv", "weight", "mask")}
    if "grad_out" in inp:
        d["grad_out"] = to_dev(inp["grad_out"], dev)
    return d


def run_fwd(dx, n=None, stream=None):
    x = dx["x"]
    n = x.shape[0] if n is None else n
    out = poison(torch.empty_like(x))
    saved = poison(torch.empty((x.shape[0], 4, 4), dtype=torch.float32, device=x.device))
    eg.engram_gate_fwd(x, dx["kv"], dx["weight"], dx["mask"], out, saved, n, stream=stream)
    return out, saved


def alloc_bwd(x, kv, n):
    dev = x.device
    gx = poison(torch.empty_like(x))
    gkv = poison(torch.empty_like(kv))
    gw = poison(torch.empty((4, D), dtype=torch.float32, device=dev))
    ws = poison(torch.empty(eg.engram_gate_bwd_workspace_bytes(n), dtype=torch.uint8, device=dev))
    return gx, gkv, gw, ws


def run_bwd(dx, saved, n=None, stream=None):
    x, kv = dx["x"], dx["kv"]
    n = x.shape[0] if n is None else n
    gx, gkv, gw, ws = alloc_bwd(x, kv, n)
    eg.engram_gate_bwd(x, kv, dx["weight"], saved, dx["grad_out"], gx, gkv, gw, ws, n, stream=stream)
    return gx, gkv, gw
