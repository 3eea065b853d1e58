"""Invariances of GateConv's definition, checked on the fp64 oracle over random
sizes, inputs and scales (hypothesis).

The relations follow from the structure of the op ("Engram Operators",
GateConv section: RMSNorm gating of H and k with one weight, a causal
four-tap depthwise conv of the RMS-normalised gated value, SiLU and the gated
value as residual), so none of the expected values comes from the oracle.
With eps = 0 every RMS norm is exactly invariant to scaling its row:
  - H row times 2^a, k row times 2^b: alpha, vhat, Y, rrms_v unchanged,
    rrms_h and rrms_k times 2^-a and 2^-b, dH and dk times 2^-a and 2^-b,
    the weight gradients and dv unchanged;
  - v row times 2^e: u (the RMS-normalised vhat) is unchanged, so c and
    SiLU(c) = Y - vhat are, vhat and rrms_v scale by 2^e and 2^-e; the
    gate's gradient reaches alpha only through the residual (d alpha = <dY,
    v> per row), so dH and dk scale by 2^e, dv - alpha dY by 2^-e, and
    drms_w_v and dconv_w are unchanged;
  - H and k exchanged: the gate's logit is symmetric, so everything but the
    pairs (rrms_h, rrms_k) and (dH, dk), which swap, is unchanged;
  - rms_w_h negated: both normalised rows change sign, the logit does not;
    only drms_w_h changes, by its sign;
  - rms_w_v times 2^e and conv_w divided by 2^e (per column): the conv's
    input and weights trade the factor, c is unchanged, drms_w_v times 2^-e,
    dconv_w times 2^e;
  - sequences permuted: per-sequence outputs permuted alike, the weight
    gradients summed over sequences in another order;
  - Euler's relations, per row: <H, dH> = 0 and <k, dk> = 0 (the gate is
    invariant to scaling either row); <v, dv> = <dY, vhat> (scaling v scales
    only the residual term of Y); per column:
    rms_w_v drms_w_v = sum_i conv_w[i] dconv_w[i] (the exchange above).
"""
from __future__ import annotations

import numpy as np
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

import oracle  # noqa: E402

EPS = 0.0


@st.composite
def _case(draw):
    M = draw(st.integers(1, 3))
    T = draw(st.integers(1, 9))
    d = draw(st.sampled_from([4, 8, 16, 24]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    H, k, v, dY = (rng.standard_normal((M, T, d)) for _ in range(4))
    wh = 1.0 + 0.25 * rng.standard_normal(d)
    wv = 1.0 + 0.25 * rng.standard_normal(d)
    cw = 0.5 * rng.standard_normal((oracle.GATECONV_TAPS, d))
    return dict(H=H, k=k, v=v, dY=dY, wh=wh, wv=wv, cw=cw, rng=rng)


def _run(c):
    Y, vhat, al, rh, rk, rv = oracle.gateconv_fwd_f64(c["H"], c["k"], c["v"], c["wh"], c["wv"], c["cw"], eps=EPS)
    g = oracle.gateconv_bwd_f64(c["dY"], c["H"], c["k"], c["v"], c["wh"], c["wv"], c["cw"], vhat, al, rh, rk, rv)
    return dict(Y=Y, vhat=vhat, alpha=al, rh=rh, rk=rk, rv=rv, dH=g[0], dk=g[1], dv=g[2], dwh=g[3], dwv=g[4],
                dcw=g[5])


def _close(a, b, rel=1e-11):
    scale = max(np.max(np.abs(b)), 1e-300)
    assert np.max(np.abs(a - b)) <= rel * scale, np.max(np.abs(a - b)) / scale


def _same(r, s, keys):
    for key in keys:
        _close(s[key], r[key])


@settings(max_examples=60, deadline=None)
@given(_case())
def test_row_scales_of_H_and_k(c):
    r = _run(c)
    M, T, d = c["H"].shape
    a = c["rng"].integers(-6, 7, size=(M, T))
    b = c["rng"].integers(-6, 7, size=(M, T))
    sa, sb = 2.0 ** a, 2.0 ** b
    s = _run(dict(c, H=c["H"] * sa[..., None], k=c["k"] * sb[..., None]))
    _same(r, s, ("alpha", "vhat", "Y", "rv", "dv", "dwh", "dwv", "dcw"))
    _close(s["rh"], r["rh"] / sa)
    _close(s["rk"], r["rk"] / sb)
    _close(s["dH"] * sa[..., None], r["dH"])
    _close(s["dk"] * sb[..., None], r["dk"])


@settings(max_examples=60, deadline=None)
@given(_case())
def test_row_scales_of_v(c):
    r = _run(c)
    M, T, d = c["H"].shape
    sc = 2.0 ** c["rng"].integers(-6, 7, size=(M, T))
    s = _run(dict(c, v=c["v"] * sc[..., None]))
    _same(r, s, ("alpha", "rh", "rk", "dwv", "dcw"))
    _close(s["vhat"], r["vhat"] * sc[..., None])
    _close(s["rv"], r["rv"] / sc)
    # SiLU(c) = Y - vhat, to the rounding of the subtraction's operands
    big = max(np.max(np.abs(a)) for a in (s["Y"], s["vhat"], r["Y"], r["vhat"]))
    assert np.max(np.abs((s["Y"] - s["vhat"]) - (r["Y"] - r["vhat"]))) <= 1e-11 * big
    _close(s["dH"], r["dH"] * sc[..., None])
    _close(s["dk"], r["dk"] * sc[..., None])
    res = r["alpha"][..., None] * c["dY"]            # the residual's share of dv
    _close((s["dv"] - res) * sc[..., None], r["dv"] - res)


@settings(max_examples=60, deadline=None)
@given(_case())
def test_exchange_of_H_and_k(c):
    r = _run(c)
    s = _run(dict(c, H=c["k"], k=c["H"]))
    _same(r, s, ("alpha", "vhat", "Y", "rv", "dv", "dwh", "dwv", "dcw"))
    _close(s["rh"], r["rk"])
    _close(s["rk"], r["rh"])
    _close(s["dH"], r["dk"])
    _close(s["dk"], r["dH"])


@settings(max_examples=60, deadline=None)
@given(_case())
def test_negated_rms_w_h(c):
    r = _run(c)
    s = _run(dict(c, wh=-c["wh"]))
    _same(r, s, ("alpha", "vhat", "Y", "rh", "rk", "rv", "dH", "dk", "dv", "dwv", "dcw"))
    _close(s["dwh"], -r["dwh"])


@settings(max_examples=60, deadline=None)
@given(_case())
def test_rms_w_v_and_conv_w_trade_a_factor(c):
    r = _run(c)
    e = 2.0 ** c["rng"].integers(-4, 5, size=c["wv"].shape)
    s = _run(dict(c, wv=c["wv"] * e, cw=c["cw"] / e))
    _same(r, s, ("alpha", "vhat", "Y", "rh", "rk", "rv", "dH", "dk", "dv", "dwh"))
    _close(s["dwv"] * e, r["dwv"])
    _close(s["dcw"] / e, r["dcw"])


@settings(max_examples=40, deadline=None)
@given(_case())
def test_sequence_permutation(c):
    M = c["H"].shape[0]
    perm = c["rng"].permutation(M)
    r = _run(c)
    s = _run(dict(c, H=c["H"][perm], k=c["k"][perm], v=c["v"][perm], dY=c["dY"][perm]))
    for key in ("Y", "vhat", "alpha", "rh", "rk", "rv", "dH", "dk", "dv"):
        assert np.array_equal(s[key], r[key][perm]), key
    _same(r, s, ("dwh", "dwv", "dcw"))


def _orth(x, y, extra=None):
    """<x, y> per row (last axis) is zero, or equals `extra`, to rounding."""
    lhs = np.sum(x * y, axis=-1)
    mag = np.sum(np.abs(x * y), axis=-1)
    rhs = 0.0 if extra is None else np.sum(extra[0] * extra[1], axis=-1)
    if extra is not None:
        mag = mag + np.sum(np.abs(extra[0] * extra[1]), axis=-1)
    assert np.all(np.abs(lhs - rhs) <= 1e-11 * mag + 1e-300), np.max(np.abs(lhs - rhs) / np.maximum(mag, 1e-300))


@settings(max_examples=60, deadline=None)
@given(_case())
def test_euler_relations(c):
    r = _run(c)
    _orth(c["H"], r["dH"])
    _orth(c["k"], r["dk"])
    _orth(c["v"], r["dv"], extra=(c["dY"], r["vhat"]))
    # per column: rms_w_v drms_w_v = sum_i conv_w[i] dconv_w[i]
    lhs = c["wv"] * r["dwv"]
    rhs = np.sum(c["cw"] * r["dcw"], axis=0)
    mag = np.abs(lhs) + np.sum(np.abs(c["cw"] * r["dcw"]), axis=0)
    assert np.all(np.abs(lhs - rhs) <= 1e-11 * mag + 1e-300)
    # the relations are not empty: the gradients do move
    assert np.any(r["dH"] != 0.0) and np.any(r["dk"] != 0.0) and np.any(r["dwv"] != 0.0)
