"""The Python binding checks tensor arguments before anything reaches the C ABI.

The library sees raw pointers only, so a tensor of the wrong element type,
shorter than the call's N rows, or a workspace below the required size would
become out-of-bounds device accesses.  Each case here builds the arguments as
meta tensors (shapes and dtypes, no memory), breaks one, and checks that the
binding raises ValueError naming it -- with the library replaced by a stub
that fails the test if any entry point is called.  Correct arguments that are
not on a GPU are refused too.
"""
from __future__ import annotations

import pytest
import torch

import memory_bound_engram_amd as eg


class _NoCalls:
    """Stands in for the ctypes library: any compute call fails the test;
    the pure host size functions still answer."""

    def __init__(self, real):
        self._real = real

    def __getattr__(self, name):
        if name.endswith("workspace_bytes") or name in ("engram_status_string", "engram_last_hip_error"):
            return getattr(self._real, name)

        def _fail(*a, **k):
            raise AssertionError(f"{name} reached the library with invalid arguments")
        return _fail


@pytest.fixture(autouse=True)
def no_library_calls(monkeypatch):
    monkeypatch.setattr(eg, "lib", _NoCalls(eg.lib))


def meta(shape, dtype):
    return torch.empty(shape, dtype=dtype, device="meta")


def gate_fwd_args(n):
    return dict(x=meta((n, 4, 5120), torch.bfloat16), kv=meta((n, 25600), torch.bfloat16),
                weight=meta((4, 5120), torch.float32), mask=meta((n,), torch.bool),
                out=meta((n, 4, 5120), torch.bfloat16), saved=meta((n, 4, 4), torch.float32))


def gate_bwd_args(n):
    return dict(x=meta((n, 4, 5120), torch.bfloat16), kv=meta((n, 25600), torch.bfloat16),
                weight=meta((4, 5120), torch.float32), saved=meta((n, 4, 4), torch.float32),
                grad_out=meta((n, 4, 5120), torch.bfloat16), grad_x=meta((n, 4, 5120), torch.bfloat16),
                grad_kv=meta((n, 25600), torch.bfloat16), grad_weight=meta((4, 5120), torch.float32),
                workspace=meta((eg.engram_gate_bwd_workspace_bytes(n),), torch.uint8))


def test_correct_meta_arguments_are_refused_only_for_their_device():
    with pytest.raises(ValueError, match="x: on meta.*GPU"):
        eg.engram_gate_fwd(**gate_fwd_args(64), N=64)
    with pytest.raises(ValueError, match="x: on meta.*GPU"):
        eg.engram_gate_bwd(**gate_bwd_args(64), N=64)


def test_cpu_tensors_are_refused():
    a = {k: torch.empty(v.shape, dtype=v.dtype) for k, v in gate_fwd_args(2).items()}
    with pytest.raises(ValueError, match="GPU"):
        eg.engram_gate_fwd(**a, N=2)


@pytest.mark.parametrize("name,shape,dtype,msg", [
    ("x", (63, 4, 5120), torch.bfloat16, "x: .* needs at least"),
    ("x", (64, 4, 5120), torch.float32, "x: dtype float32"),
    ("kv", (64, 20480), torch.bfloat16, "kv: .* needs at least"),
    ("weight", (4, 5120), torch.bfloat16, "weight: dtype bfloat16"),
    ("mask", (63,), torch.bool, "mask: .* needs at least"),
    ("mask", (64,), torch.int32, "mask: dtype int32"),
    ("out", (64, 4, 2560), torch.bfloat16, "out: .* needs at least"),
    ("saved", (64, 4, 4), torch.float16, "saved: dtype float16"),
])
def test_forward_rejects_bad_tensor(name, shape, dtype, msg):
    a = gate_fwd_args(64)
    a[name] = meta(shape, dtype)
    with pytest.raises(ValueError, match=msg):
        eg.engram_gate_fwd(**a, N=64)


def test_forward_n_larger_than_the_tensors():
    a = gate_fwd_args(64)
    with pytest.raises(ValueError, match="needs at least"):
        eg.engram_gate_fwd(**a, N=128)


@pytest.mark.parametrize("name,shape,dtype,msg", [
    ("saved", (64, 4, 3), torch.float32, "saved: .* needs at least"),
    ("grad_out", (64, 4, 5120), torch.float16, "grad_out: dtype float16"),
    ("grad_x", (32, 4, 5120), torch.bfloat16, "grad_x: .* needs at least"),
    ("grad_kv", (64, 25600), torch.float32, "grad_kv: dtype float32"),
    ("grad_weight", (4, 5119), torch.float32, "grad_weight: .* needs at least"),
    ("workspace", (1000,), torch.uint8, "workspace: 1000 bytes"),
])
def test_backward_rejects_bad_tensor(name, shape, dtype, msg):
    a = gate_bwd_args(64)
    a[name] = meta(shape, dtype)
    with pytest.raises(ValueError, match=msg):
        eg.engram_gate_bwd(**a, N=64)


def test_backward_workspace_sized_for_a_smaller_n():
    a = gate_bwd_args(128)
    a["workspace"] = meta((eg.engram_gate_bwd_workspace_bytes(64),), torch.uint8)
    with pytest.raises(ValueError, match="workspace: .* bytes, the call needs"):
        eg.engram_gate_bwd(**a, N=128)


def test_backward_with_norm_weights_checks_the_extra_tensors():
    a = gate_bwd_args(64)
    extra = dict(wh=meta((4, 5120), torch.bfloat16), we=meta((4, 5120), torch.float32),
                 grad_wh=meta((4, 5120), torch.float32), grad_we=meta((4, 5120), torch.float32))
    with pytest.raises(ValueError, match="we: dtype float32"):
        eg.engram_gate_bwd_with_norm_weights(**a, **extra, N=64)


def test_fused_weight_checks_sizes():
    with pytest.raises(ValueError, match="we: .* needs at least"):
        eg.engram_fused_weight(meta((4, 5120), torch.bfloat16), meta((4, 100), torch.bfloat16),
                               meta((4, 5120), torch.float32))


def gc_args(M, T, d):
    t = lambda: meta((M, T, d), torch.bfloat16)  # noqa: E731
    s = lambda: meta((M, T), torch.float32)  # noqa: E731
    return dict(H=t(), k=t(), v=t(), rms_w_h=meta((d,), torch.float32), rms_w_v=meta((d,), torch.float32),
                conv_w=meta((4, d), torch.float32), Y=t(), vhat=t(), alpha=s(), rrms_h=s(), rrms_k=s(), rrms_v=s())


@pytest.mark.parametrize("name,shape,dtype,msg", [
    ("k", (2, 9, 256), torch.bfloat16, "k: .* needs at least"),
    ("conv_w", (3, 512), torch.float32, "conv_w: .* needs at least"),
    ("alpha", (2, 9), torch.bfloat16, "alpha: dtype bfloat16"),
    ("Y", (2, 9, 512), torch.float32, "Y: dtype float32"),
])
def test_gateconv_forward_rejects_bad_tensor(name, shape, dtype, msg):
    a = gc_args(2, 9, 512)
    a[name] = meta(shape, dtype)
    with pytest.raises(ValueError, match=msg):
        eg.engram_gateconv_fwd(**a)


def test_gateconv_backward_rejects_a_short_workspace():
    M, T, d = 2, 9, 512
    f = gc_args(M, T, d)
    t = lambda: meta((M, T, d), torch.bfloat16)  # noqa: E731
    args = dict(dY=t(), H=f["H"], k=f["k"], v=f["v"], rms_w_h=f["rms_w_h"], rms_w_v=f["rms_w_v"],
                conv_w=f["conv_w"], vhat=f["vhat"], alpha=f["alpha"], rrms_h=f["rrms_h"], rrms_k=f["rrms_k"],
                rrms_v=f["rrms_v"], dH=t(), dk=t(), dv=t(), drms_w_h=meta((d,), torch.float32),
                drms_w_v=meta((d,), torch.float32), dconv_w=meta((4, d), torch.float32),
                workspace=meta((16,), torch.uint8))
    with pytest.raises(ValueError, match="workspace: 16 bytes"):
        eg.engram_gateconv_bwd(**args)
    args["workspace"] = meta((eg.engram_gateconv_bwd_workspace_bytes(M, T, d),), torch.uint8)
    args["dv"] = meta((M, T, d), torch.float32)
    with pytest.raises(ValueError, match="dv: dtype float32"):
        eg.engram_gateconv_bwd(**args)


def test_noalloc_backward_checks_tensors():
    a = gate_bwd_args(64)
    del a["workspace"]
    a["grad_kv"] = meta((64, 25599), torch.bfloat16)
    with pytest.raises(ValueError, match="grad_kv: .* needs at least"):
        eg.engram_gate_bwd_noalloc(**a, N=64)
