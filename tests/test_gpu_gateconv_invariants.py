"""Exact invariances of GateConv, checked on the device against the device.

Each test runs libengram's GateConv twice, on inputs and on an exactly
transformed copy, and compares the two results bit for bit, without the
oracle.  The relations follow from the op's structure ("Engram Operators",
GateConv section: one RMSNorm weight for H and k, the RMS-normalised gated
value through a depthwise conv) and hold exactly in the kernels' fp32
arithmetic because each transform is exact and commutes with rounding:

  rms_w_h negated:   the kernels use rms_w_h through its square and, in the
                     rms_w_h gradient, linearly: every output is unchanged and
                     drms_w_h is negated (round-to-nearest-even is symmetric).
  rms_w_v times 2^e, conv_w over 2^e (per column): the conv's input u and its
                     taps trade the factor, c is the same number, so the
                     forward and dH, dk, dv are unchanged bit for bit; the
                     conv_w gradient (w_v times a sum) scales by 2^e and the
                     rms_w_v gradient (conv_w against the same sums) by 2^-e.
  eps = 0, H rows times 2^a, k rows times 2^b: the sums of squares scale by
                     4^a and 4^b, so rrms_h and rrms_k scale by 2^-a and 2^-b
                     (a reciprocal square root keeps the exponent's parity);
                     alpha, Y, vhat, rrms_v are unchanged; dH and dk scale by
                     2^-a and 2^-b; dv and every weight gradient unchanged.

Shapes cover each column map of the kernels (d = 5120: 512 x 10; 4608: 512 x
9; 2560 and 1536: the backward's 256 x 10 and 768 x 2) and a two-level weight
gradient sum (d = 512 over 16,384 rows: 1024 workgroups).
"""
from __future__ import annotations

import numpy as np
import pytest

import synth
from test_gpu_gateconv import run_bwd, run_fwd

pytestmark = pytest.mark.gpu

SHAPES = [(2, 1500, 5120), (1, 900, 4608), (2, 700, 2560), (4, 1000, 1536), (8, 2048, 512)]
SAVED = ("vhat", "alpha", "rh", "rk", "rv")


def _bits(a):
    return a.view(np.uint32) if a.dtype == np.float32 else a


def _eq(a, b, what):
    assert np.array_equal(_bits(a), _bits(b)), f"{what}: {np.count_nonzero(_bits(a) != _bits(b))} elements differ"


def _both(inp, gpu, eps=1e-6):
    f = run_fwd(inp, gpu, eps=eps)
    b = run_bwd(inp, {k: f[k] for k in SAVED}, gpu)
    return f, b


def _bf16_rows_scaled(bits, k):
    """bf16 rows [..., d] times 2^k (k per row), exactly (normal values only)."""
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    g = f * (2.0 ** k).astype(np.float32)[..., None]
    out = (g.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((out.astype(np.uint32) << 16).view(np.float32), g), "scale not exact in bf16"
    return out


@pytest.mark.parametrize("M,T,d", SHAPES)
def test_negated_rms_w_h(gpu, M, T, d):
    inp = synth.gateconv_inputs(M, T, d, seed=41, edge=True)
    fa, ba = _both(inp, gpu)
    fb, bb = _both(dict(inp, wh=-inp["wh"]), gpu)
    for key in ("Y", "vhat", "alpha", "rh", "rk", "rv"):
        _eq(fb[key], fa[key], key)
    for key in ("dH", "dk", "dv", "dwv", "dcw"):
        _eq(bb[key], ba[key], key)
    _eq(bb["dwh"], -ba["dwh"], "drms_w_h negated")


@pytest.mark.parametrize("M,T,d", SHAPES)
def test_rms_w_v_and_conv_w_trade_a_power_of_two(gpu, M, T, d):
    inp = synth.gateconv_inputs(M, T, d, seed=42, edge=True)
    e = np.random.default_rng(42).integers(-4, 5, size=d)
    sc = (2.0 ** e).astype(np.float32)
    wv2, cw2 = inp["wv"] * sc, inp["cw"] / sc
    assert np.array_equal(wv2 / sc, inp["wv"]) and np.array_equal(cw2 * sc, inp["cw"])
    fa, ba = _both(inp, gpu)
    fb, bb = _both(dict(inp, wv=wv2, cw=cw2), gpu)
    for key in ("Y", "vhat", "alpha", "rh", "rk", "rv"):
        _eq(fb[key], fa[key], key)
    for key in ("dH", "dk", "dv", "dwh"):
        _eq(bb[key], ba[key], key)
    _eq(bb["dcw"], ba["dcw"] * sc, "dconv_w times 2^e")
    _eq(bb["dwv"], ba["dwv"] / sc, "drms_w_v times 2^-e")


@pytest.mark.parametrize("M,T,d", SHAPES)
def test_row_scales_of_H_and_k_at_eps_zero(gpu, M, T, d):
    # no edge rows: a zero row has no RMS at eps = 0
    inp = synth.gateconv_inputs(M, T, d, seed=43)
    rng = np.random.default_rng(43)
    a = rng.integers(-5, 6, size=(M, T))
    b = rng.integers(-5, 6, size=(M, T))
    H2, k2 = _bf16_rows_scaled(inp["H"], a), _bf16_rows_scaled(inp["k"], b)
    fa, ba = _both(inp, gpu, eps=0.0)
    fb, bb = _both(dict(inp, H=H2, k=k2), gpu, eps=0.0)
    sa, sb = (2.0 ** -a).astype(np.float32), (2.0 ** -b).astype(np.float32)
    _eq(fb["rh"], fa["rh"] * sa, "rrms_h times 2^-a")
    _eq(fb["rk"], fa["rk"] * sb, "rrms_k times 2^-b")
    for key in ("Y", "vhat", "alpha", "rv"):
        _eq(fb[key], fa[key], key)
    _eq(bb["dH"], _bf16_rows_scaled(ba["dH"], -a), "dH times 2^-a")
    _eq(bb["dk"], _bf16_rows_scaled(ba["dk"], -b), "dk times 2^-b")
    for key in ("dv", "dwh", "dwv", "dcw"):
        _eq(bb[key], ba[key], key)
