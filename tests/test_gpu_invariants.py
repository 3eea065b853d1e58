"""Exact invariants of the gate, checked on the device against the device.

Each test runs libengram twice, on inputs and on an exactly transformed copy
of them, and compares the two results without the oracle.  The relations
follow from the definition ("Engram saved-state gate", semantics paragraph)
and hold bit for bit in fp32 arithmetic because the transforms are exact and
the kernels treat every stream, and every power-of-two scale, alike:

  key negation:   dot -> -dot exactly, rstd_X and rstd_key unchanged, gate ->
                  1 - gate (to rounding); in the backward grad_key is unchanged
                  and grad_weight negated (to the rounding of gate (1 - gate),
                  large in relative terms where the gate saturates).
  2^a X, 2^b key: rstd_X -> 2^-a rstd_X and rstd_key -> 2^-b rstd_key exactly,
                  dot and gate unchanged bit for bit (x^ and k^ are the same
                  fp32 numbers); grad_key -> 2^-b grad_key and grad_weight
                  unchanged, bit for bit, given the same saved gate and dot.
  stream order:   permuting the streams of X and grad_out, the key blocks and
                  the weight rows permutes out, saved, grad_x, grad_key and
                  grad_weight bit for bit; the shared value's gradient sums
                  the four stream terms in another order (within the error
                  bound of a reordered four-term fp32 sum and a bf16 cast).

eps (1e-20) is far below half an ulp of the mean squares of these rows, so it
drops out of every sum it enters, as the scale relation needs.
"""
from __future__ import annotations

import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

D = 5120


def _bf16_scaled(bits: np.ndarray, k: int) -> np.ndarray:
    """bf16 bit patterns times 2^k, exactly (normal values in, normal values out)."""
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    g = f * np.float32(2.0 ** k)
    out = (g.view(np.uint32) >> 16).astype(np.uint16)
    back = (out.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(back, g), "scale not exact in bf16"
    return out


def _run(inp, gpu, saved=None):
    """Forward, then the backward on `saved` (default: this forward's own)."""
    import torch
    from gpu_util import dev_inputs, f32, run_bwd, run_fwd, to_dev, u16
    d = dev_inputs(inp, gpu)
    out, sv = run_fwd(d)
    gx, gkv, gw = run_bwd(d, sv if saved is None else to_dev(saved, gpu))
    torch.cuda.synchronize()
    return {"out": u16(out), "saved": f32(sv), "dx": u16(gx), "dkv": u16(gkv), "dw": f32(gw)}


def _bf16_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_key_negation(gpu):
    n = 4160  # the backward's two-round partition (65 rows)
    inp = synth.host_inputs(n, seed=31, p=0.8, grad=True)
    neg = dict(inp)
    kv = inp["kv"].copy()
    kv[:, :4 * D] ^= np.uint16(0x8000)  # the four keys; the shared value stays
    neg["kv"] = kv
    a, b = _run(inp, gpu), _run(neg, gpu)
    sa, sb = a["saved"], b["saved"]
    assert np.array_equal(sb[..., 1], -sa[..., 1]), "dot not negated exactly"
    assert np.array_equal(sb[..., 2].view(np.uint32), sa[..., 2].view(np.uint32)), "rstd_X changed"
    assert np.array_equal(sb[..., 3].view(np.uint32), sa[..., 3].view(np.uint32)), "rstd_key changed"
    m = inp["mask"].astype(bool)
    assert np.all(sa[~m, :, 0] == 0) and np.all(sb[~m, :, 0] == 0)
    gap = np.abs(sb[m, :, 0].astype(np.float64) - (1.0 - sa[m, :, 0].astype(np.float64)))
    assert gap.max() <= 2.0 ** -22, f"gate(-k) vs 1 - gate(k): {gap.max():.3e}"
    # backward: grad_key unchanged, delta(-k) = delta(k) up to the gate's
    # rounding.  Where the gate saturates (|dot| runs to ~300 on these rows,
    # so gate is within 1e-7 of 0 or 1) fp32 gets gate (1 - gate) from a
    # cancellation on one side and directly on the other: a large relative
    # but tiny absolute difference in delta, hence the bound's second term.
    ka = _bf16_f64(a["dkv"][:, :4 * D]).reshape(n, 4, D)
    kb = _bf16_f64(b["dkv"][:, :4 * D]).reshape(n, 4, D)
    scale = np.abs(ka).max(axis=(0, 2), keepdims=True)
    bad = np.abs(kb - ka) > 2.0 ** -7 * np.abs(ka) + 1e-6 * scale
    assert not bad.any(), f"grad_key moved on {np.count_nonzero(bad)} elements"
    dw_a, dw_b = a["dw"].astype(np.float64), b["dw"].astype(np.float64)
    assert np.max(np.abs(dw_b + dw_a)) <= 1e-5 * np.max(np.abs(dw_a)), "grad_weight not negated"
    sat = np.minimum(sa[m, :, 0], 1.0 - sa[m, :, 0]) < 1e-6
    print(f"key negation: gate gap {gap.max():.2e}; {np.count_nonzero(sat)} saturated (token, stream) rows; "
          f"grad_key max |diff| / stream max {np.max(np.abs(kb - ka) / scale):.2e}")


@pytest.mark.parametrize("a,b", [(3, -2), (-5, 4)])
def test_power_of_two_scaling(gpu, a, b):
    n = 8192
    inp = synth.host_inputs(n, seed=32, p=0.9, grad=True)
    sc = dict(inp)
    sc["x"] = _bf16_scaled(inp["x"], a)
    kv = inp["kv"].copy()
    kv[:, :4 * D] = _bf16_scaled(kv[:, :4 * D], b)
    sc["kv"] = kv
    r0 = _run(inp, gpu)
    r1 = _run(sc, gpu, saved=None)
    s0, s1 = r0["saved"], r1["saved"]
    for f, name in ((0, "gate"), (1, "dot")):
        assert np.array_equal(s1[..., f].view(np.uint32), s0[..., f].view(np.uint32)), f"{name} changed"
    assert np.array_equal(s1[..., 2], s0[..., 2] * np.float32(2.0 ** -a)), "rstd_X not scaled exactly"
    assert np.array_equal(s1[..., 3], s0[..., 3] * np.float32(2.0 ** -b)), "rstd_key not scaled exactly"
    # the backward sees the same gate and dot, and x^ and k^ are the same numbers
    want_dk = _bf16_scaled(r0["dkv"][:, :4 * D], -b)
    assert np.array_equal(r1["dkv"][:, :4 * D], want_dk), "grad_key not scaled exactly"
    assert np.array_equal(r1["dw"].view(np.uint32), r0["dw"].view(np.uint32)), "grad_weight changed"
    assert np.array_equal(r1["dkv"][:, 4 * D:], r0["dkv"][:, 4 * D:]), "grad_value changed"


def test_stream_permutation(gpu):
    n = 8192
    perm = np.array([2, 0, 3, 1])
    inp = synth.host_inputs(n, seed=33, p=0.7, grad=True)
    pm = dict(inp)
    pm["x"] = np.ascontiguousarray(inp["x"][:, perm])
    pm["grad_out"] = np.ascontiguousarray(inp["grad_out"][:, perm])
    keys = inp["kv"][:, :4 * D].reshape(n, 4, D)[:, perm].reshape(n, 4 * D)
    pm["kv"] = np.ascontiguousarray(np.concatenate([keys, inp["kv"][:, 4 * D:]], axis=1))
    pm["weight"] = np.ascontiguousarray(inp["weight"][perm])
    a, b = _run(inp, gpu), _run(pm, gpu)
    assert np.array_equal(b["out"], a["out"][:, perm]), "out"
    assert np.array_equal(b["saved"].view(np.uint32), a["saved"][:, perm].view(np.uint32)), "saved"
    assert np.array_equal(b["dx"], a["dx"][:, perm]), "grad_x"
    dk_a = a["dkv"][:, :4 * D].reshape(n, 4, D)
    dk_b = b["dkv"][:, :4 * D].reshape(n, 4, D)
    assert np.array_equal(dk_b, dk_a[:, perm]), "grad_key"
    assert np.array_equal(b["dw"].view(np.uint32), a["dw"][perm].view(np.uint32)), "grad_weight"
    # grad_value: the four fp32 terms gate_s G_s summed in another order.  Two
    # orders differ by at most 2 x 3 u sum_s |gate_s G_s| (u = 2^-24) before
    # each side's bf16 rounding (half an ulp, at most 2^-8 |value|); where the
    # terms cancel the sign may differ, so the bound is absolute.
    va, vb = _bf16_f64(a["dkv"][:, 4 * D:]), _bf16_f64(b["dkv"][:, 4 * D:])
    mag = np.zeros((n, D))
    for s_ in range(4):
        mag += np.abs(a["saved"][:, s_, 0:1].astype(np.float64)) * np.abs(_bf16_f64(inp["grad_out"][:, s_]))
    bound = 6 * 2.0 ** -24 * mag + 2.0 ** -8 * (np.abs(va) + np.abs(vb))
    over = np.abs(vb - va) > bound
    assert not over.any(), f"grad_value off on {np.count_nonzero(over)} elements"
    print(f"stream permutation: grad_value differs on {np.count_nonzero(va != vb)} of {va.size} elements, "
          f"max |diff| / bound {np.max(np.abs(vb - va) / np.maximum(bound, 1e-300)):.2f}")
