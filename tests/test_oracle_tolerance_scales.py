"""Pins of the oracle's tolerance scales.

Besides the method's values, the oracle emits magnitudes that set the width
of every elementwise parity bar: for the gate, the dot's conditioning
A = sum_j |x^_j w_j k^_j| and d gate / d dot (forward), and the sums of
|terms| of grad_x, grad_kv and grad_weight (backward); for GateConv, a
first-order magnitude of every output.  A mistake there (a factor 1000, a
dropped term) would widen or narrow every bar while the method's own pins
still pass, so these tests fix the magnitudes from two sides:

* a plain numpy recomputation, written here from the construction each
  magnitude states, on small cases (d = 16, and a few d = 5120 rows on the
  storage-type entry points), equal to the oracle's to rounding -- this bounds
  them from above as well as below;
* special cases where the magnitude must equal |value| exactly because every
  term of the value has the same sign (so the sum of |terms| is the |sum|),
  tied to values that the other pin files check against finite differences:
  A = dot when the key row equals the X row and the weight is positive;
  grad_x, grad_key, grad_value and grad_weight at coordinates where all their
  terms share a sign; and d gate / d dot against the ratio of central
  differences of the oracle's own gate and dot.

Reference: "Engram saved-state gate", semantics paragraph (the FP32
reductions whose evaluation error these magnitudes scale), and "Engram
Operators", GateConv section, for the GateConv outputs.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth
from numerics import bf16_to_f64

EPS = float(np.float32(1e-20))
CLAMP = float(np.float32(1e-6))
RT = 1e-12  # agreement to rounding (fp64 sums in different orders)


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


# --------------------------------------------------------------------------
# the gate: independent recomputation
# --------------------------------------------------------------------------

def np_gate_fwd_scales(x, kv, w, mask):
    """(A, d gate/d dot) from the definition: x [n,4,d], kv [n,5d], w [4,d] fp64."""
    n, S, d = x.shape
    k = kv[:, :S * d].reshape(n, S, d)
    rx = 1.0 / np.sqrt((x * x).sum(-1) / d + EPS)
    rk = 1.0 / np.sqrt((k * k).sum(-1) / d + EPS)
    terms = (x * rx[..., None]) * w[None] * (k * rk[..., None])
    dot = terms.sum(-1)
    A = np.abs(terms).sum(-1)
    z = np.sign(dot) * np.sqrt(np.maximum(np.abs(dot), CLAMP))
    g = sigmoid(z)
    with np.errstate(divide="ignore"):
        slope = np.where(np.abs(dot) >= CLAMP, g * (1 - g) / (2 * np.sqrt(np.abs(dot))), 0.0)
    slope = np.where((mask != 0)[:, None], slope, 0.0)
    return A, slope


def np_gate_bwd_scales(x, kv, w, saved, G):
    """(mag_dx, mag_dkv, mag_dw): sums of |terms| with |delta| bounded through
    sum_j |G_j v_j| (the grad-of-gate reduction cancels on the device)."""
    n, S, d = x.shape
    k = kv[:, :S * d].reshape(n, S, d)
    v = kv[:, S * d:]
    gate, dot, rx, rk = (saved[..., i] for i in range(4))
    dgabs = np.abs(G * v[:, None, :]).sum(-1)
    with np.errstate(divide="ignore", invalid="ignore"):
        dmag = np.where(np.abs(dot) >= CLAMP, dgabs * gate * (1 - gate) / (2 * np.sqrt(np.abs(dot))), 0.0)
    xh, kh = x * rx[..., None], k * rk[..., None]
    ad = np.abs(dot)[..., None]
    mdx = np.abs(G) + (dmag * rx)[..., None] * (np.abs(w[None] * kh) + ad * np.abs(xh) / d)
    mdk = (dmag * rk)[..., None] * (np.abs(w[None] * xh) + ad * np.abs(kh) / d)
    mdv = np.abs(gate[..., None] * G).sum(1)
    mdkv = np.concatenate([mdk.reshape(n, S * d), mdv], axis=1)
    mdw = (dmag[..., None] * np.abs(xh * kh)).sum(0)
    return mdx, mdkv, mdw


def _small_f64_case(n=3, d=16, seed=5):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 4, d))
    kv = rng.standard_normal((n, 5 * d))
    w = 1.0 + 0.1 * rng.standard_normal((4, d))
    G = rng.standard_normal((n, 4, d))
    mask = np.ones(n, np.uint8)
    mask[1] = 0                               # a masked token
    kv[2, 1 * d:2 * d] *= 2.0 ** -64          # token 2, stream 1 on the clamp path
    return x, kv, w, mask, G


def test_gate_forward_scales_match_numpy_f64():
    x, kv, w, mask, _ = _small_f64_case()
    _, saved, aux = oracle.fwd_f64(x, kv, w, mask, aux=True)
    A, slope = np_gate_fwd_scales(x, kv, w, mask)
    np.testing.assert_allclose(aux[..., 0], A, rtol=RT, atol=0)
    np.testing.assert_allclose(aux[..., 1], slope, rtol=RT, atol=0)
    assert np.all(aux[1, :, 1] == 0.0)        # masked token: no gate slope
    assert aux[2, 1, 1] == 0.0                # clamp path: no gate slope
    assert np.all(aux[..., 0] >= np.abs(saved[..., 1]))   # A >= |dot|


def test_gate_backward_scales_match_numpy_f64():
    x, kv, w, mask, G = _small_f64_case()
    _, saved = oracle.fwd_f64(x, kv, w, mask)
    dx, dkv, dw, mdx, mdkv, mdw = oracle.bwd_f64(x, kv, w, saved, G, mags=True)
    rdx, rdkv, rdw = np_gate_bwd_scales(x, kv, w, saved, G)
    np.testing.assert_allclose(mdx, rdx, rtol=RT, atol=0)
    np.testing.assert_allclose(mdkv, rdkv, rtol=RT, atol=0)
    np.testing.assert_allclose(mdw, rdw, rtol=RT, atol=0)
    # magnitudes bound the values they scale
    assert np.all(mdx >= np.abs(dx) * (1 - RT))
    assert np.all(mdkv >= np.abs(dkv) * (1 - RT))
    assert np.all(mdw >= np.abs(dw) * (1 - RT))


def test_gate_scales_match_numpy_storage_types():
    """The storage-type entry points (the ones the parity tests use) at
    d = 5120: a few rows with a masked token and a clamp-path stream."""
    n = 3
    inp = synth.host_inputs(n, seed=17, p=1.0, grad=True)
    x16, kv16 = inp["x"], inp["kv"].copy()
    kv16[0, 2 * 5120:3 * 5120] = 0            # token 0, stream 2: zero key (dot = 0 exactly)
    mask = np.array([1, 0, 1], np.uint8)
    w32 = inp["weight"]
    _, saved32, _, saved64, aux = oracle.fwd_bf16(x16, kv16, w32, mask, extras=True)
    x, kv, w = bf16_to_f64(x16), bf16_to_f64(kv16), w32.astype(np.float64)
    A, slope = np_gate_fwd_scales(x, kv, w, mask)
    np.testing.assert_allclose(aux[..., 0], A, rtol=RT, atol=0)
    np.testing.assert_allclose(aux[..., 1], slope, rtol=RT, atol=0)
    G = bf16_to_f64(inp["grad_out"])
    ex = oracle.bwd_bf16(x16, kv16, w32, saved32, inp["grad_out"], extras=True)
    rdx, rdkv, rdw = np_gate_bwd_scales(x, kv, w, saved32.astype(np.float64), G)
    np.testing.assert_allclose(ex[6], rdx, rtol=RT, atol=0)
    np.testing.assert_allclose(ex[7], rdkv, rtol=RT, atol=0)
    np.testing.assert_allclose(ex[8], rdw, rtol=RT, atol=0)


# --------------------------------------------------------------------------
# the gate: cases where a magnitude equals |value| (all terms of one sign)
# --------------------------------------------------------------------------

def test_dot_conditioning_equals_dot_for_identical_rows():
    """Key row = X row and weight > 0: every term x^_j w_j k^_j is >= 0, so
    A = sum |terms| equals dot itself (an upper bound as well as a lower one)."""
    rng = np.random.default_rng(3)
    n, d = 2, 64
    x = rng.standard_normal((n, 4, d))
    kv = np.concatenate([x.reshape(n, 4 * d), rng.standard_normal((n, d))], axis=1)
    w = np.abs(1.0 + 0.1 * rng.standard_normal((4, d)))
    _, saved, aux = oracle.fwd_f64(x, kv, w, np.ones(n, np.uint8), aux=True)
    np.testing.assert_allclose(aux[..., 0], saved[..., 1], rtol=RT, atol=0)


def _coherent_case(n=2, d=32, seed=9):
    """Rows where each gradient's terms share a sign on known coordinates.

    Every X and key coordinate is positive except X on the last quarter Q,
    which is negative (key positive there); weights, grad_out and the value
    are positive.  Then dot > 0, dg = sum |G v| > 0 and delta > 0, and on Q
      grad_x  = G + delta r_x (w k^ - dot x^ / d)   : all three terms >= 0
      grad_k  =     delta r_k (w x^ - dot k^ / d)   : both terms <= 0
      grad_w  = sum_t delta x^ k^                   : every term <= 0
    while grad_value = sum_s gate_s G_s has positive terms everywhere."""
    rng = np.random.default_rng(seed)
    x = np.abs(rng.standard_normal((n, 4, d))) + 0.1
    q = slice(3 * d // 4, d)
    x[:, :, q] *= -0.25                    # small, so that dot stays positive
    k = np.abs(rng.standard_normal((n, 4, d))) + 0.1
    v = np.abs(rng.standard_normal((n, d))) + 0.1
    kv = np.concatenate([k.reshape(n, 4 * d), v], axis=1)
    w = np.abs(1.0 + 0.1 * rng.standard_normal((4, d)))
    G = np.abs(rng.standard_normal((n, 4, d))) + 0.1
    return x, kv, w, G, q


def test_gate_backward_scales_equal_values_on_coherent_coordinates():
    x, kv, w, G, q = _coherent_case()
    n, _, d = x.shape
    _, saved = oracle.fwd_f64(x, kv, w, np.ones(n, np.uint8))
    assert np.all(saved[..., 1] > CLAMP)
    dx, dkv, dw, mdx, mdkv, mdw = oracle.bwd_f64(x, kv, w, saved, G, mags=True)
    np.testing.assert_allclose(mdx[:, :, q], dx[:, :, q], rtol=RT, atol=0)
    dk = dkv[:, :4 * d].reshape(n, 4, d)
    mdk = mdkv[:, :4 * d].reshape(n, 4, d)
    assert np.all(dk[:, :, q] < 0)
    np.testing.assert_allclose(mdk[:, :, q], -dk[:, :, q], rtol=RT, atol=0)
    np.testing.assert_allclose(mdkv[:, 4 * d:], dkv[:, 4 * d:], rtol=RT, atol=0)
    assert np.all(dw[:, q] < 0)
    np.testing.assert_allclose(mdw[:, q], -dw[:, q], rtol=RT, atol=0)


def test_gate_slope_matches_finite_difference_ratio():
    """d gate / d dot equals (central difference of the gate) / (central
    difference of the dot) along one X coordinate: the gate depends on X only
    through the dot.  Both differences come from the oracle's fp64 forward."""
    rng = np.random.default_rng(21)
    n, d, h = 1, 16, 1e-6
    x = rng.standard_normal((n, 4, d))
    kv = rng.standard_normal((n, 5 * d))
    w = 1.0 + 0.1 * rng.standard_normal((4, d))
    m = np.ones(n, np.uint8)
    _, saved, aux = oracle.fwd_f64(x, kv, w, m, aux=True)
    for s in range(4):
        assert abs(saved[0, s, 1]) > 1e-3      # away from the clamp and sgn kinks
        xp, xm = x.copy(), x.copy()
        xp[0, s, 3] += h
        xm[0, s, 3] -= h
        _, sp = oracle.fwd_f64(xp, kv, w, m)
        _, sm = oracle.fwd_f64(xm, kv, w, m)
        ratio = (sp[0, s, 0] - sm[0, s, 0]) / (sp[0, s, 1] - sm[0, s, 1])
        assert ratio == pytest.approx(aux[0, s, 1], rel=1e-6)


# --------------------------------------------------------------------------
# GateConv: independent recomputation of every magnitude
# --------------------------------------------------------------------------

def silu_grad(c):
    s = sigmoid(c)
    return s * (1 + c * (1 - s))


def _causal(cw, u):
    """sum_{i<4} cw[i] u[t-3+i] with zero history: u [T,d] -> [T,d]."""
    T = u.shape[0]
    out = np.zeros_like(u)
    for i in range(4):
        lag = 3 - i
        out[lag:] += cw[i] * u[:T - lag]
    return out


def _anticausal(cw, dc):
    """sum_{i<4} cw[i] dc[t+3-i] (rows past the end are zero)."""
    T = dc.shape[0]
    out = np.zeros_like(dc)
    for i in range(4):
        lead = 3 - i
        out[:T - lead] += cw[i] * dc[lead:]
    return out


def np_gateconv_fwd_mag(H, k, v, wh, wv, cw, eps):
    """magY per the construction: |SiLU(c)| + |SiLU'(c)| m(c) + |vhat| + |v| m(alpha),
    with m(alpha) = alpha (1 - alpha) sum|h^ k^| / sqrt(d), m(u) = |u| (1 + 2 m(alpha) / alpha)
    and m(c) = sum_i |cw_i| m(u_{t-3+i})."""
    M, T, d = H.shape
    sd = np.sqrt(d)
    out = np.empty_like(H)
    for m in range(M):
        rh = 1 / np.sqrt((H[m] ** 2).mean(-1) + eps)
        rk = 1 / np.sqrt((k[m] ** 2).mean(-1) + eps)
        terms = (H[m] * rh[:, None] * wh) * (k[m] * rk[:, None] * wh)
        a = sigmoid(terms.sum(-1) / sd)
        da = a * (1 - a) * np.abs(terms).sum(-1) / sd
        vhat = a[:, None] * v[m]
        rv = 1 / np.sqrt((vhat ** 2).mean(-1) + eps)
        u = vhat * rv[:, None] * wv
        with np.errstate(divide="ignore", invalid="ignore"):
            grow = np.where(a > 0, 2 * da / a, 0.0)
        um = np.abs(u) * (1 + grow)[:, None]
        c = _causal(cw, u)
        cm = _causal(np.abs(cw), um)
        out[m] = (np.abs(c * sigmoid(c)) + np.abs(silu_grad(c)) * cm + np.abs(vhat)
                  + np.abs(v[m]) * da[:, None])
    return out


def np_gateconv_bwd_mags(dY, H, k, v, wh, wv, cw, vhat, alpha, rrh, rrk, rrv):
    """(magH, magk, magv, mdwh, mdwv, mdcw) per the backward's construction."""
    M, T, d = H.shape
    sd = np.sqrt(d)
    magH, magk, magv = np.empty_like(H), np.empty_like(H), np.empty_like(H)
    mdwh, mdwv, mdcw = np.zeros(d), np.zeros(d), np.zeros((4, d))
    for m in range(M):
        a, rh, rk, rv = alpha[m][:, None], rrh[m][:, None], rrk[m][:, None], rrv[m][:, None]
        vh = vhat[m]
        u = vh * rv * wv
        c = _causal(cw, u)
        cmb = _causal(np.abs(cw), np.abs(u))
        dcm = np.abs(dY[m]) * (np.abs(silu_grad(c)) + 0.5 * cmb)
        for i in range(4):
            lag = 3 - i
            mdcw[i] += (dcm[lag:] * np.abs(u[:T - lag])).sum(0)
        dum = _anticausal(np.abs(cw), dcm)
        s1m = (dum * np.abs(wv * vh)).sum(-1, keepdims=True)
        mdwv += (dum * np.abs(vh * rv)).sum(0)
        dvhm = np.abs(dY[m]) + rv * (np.abs(wv) * dum + np.abs(vh) * rv ** 2 * s1m / d)
        dsm = (dvhm * np.abs(v[m])).sum(-1, keepdims=True) * a * (1 - a)
        pm = (np.abs(H[m] * k[m]) * wh ** 2).sum(-1, keepdims=True)
        s2m, s3m = dsm / sd * rk * pm, dsm / sd * rh * pm
        hh, kh = H[m] * rh * wh, k[m] * rk * wh
        magH[m] = rh * (np.abs(wh) * dsm * np.abs(kh) / sd + np.abs(H[m]) * rh ** 2 * s2m / d)
        magk[m] = rk * (np.abs(wh) * dsm * np.abs(hh) / sd + np.abs(k[m]) * rk ** 2 * s3m / d)
        mdwh += (dsm * (np.abs(kh * H[m] * rh) + np.abs(hh * k[m] * rk)) / sd).sum(0)
        magv[m] = dvhm * a
    return magH, magk, magv, mdwh, mdwv, mdcw


def _gc_case(M=2, T=7, d=16, seed=4):
    rng = np.random.default_rng(seed)
    H, k, v, dY = (rng.standard_normal((M, T, d)) for _ in range(4))
    wh = 1 + 0.25 * rng.standard_normal(d)
    wv = 1 + 0.25 * rng.standard_normal(d)
    cw = 0.5 * rng.standard_normal((4, d))
    v[0, 2] = 0.0          # a zero value row (alpha enters nothing downstream)
    return H, k, v, dY, wh, wv, cw


@pytest.mark.parametrize("eps", [1e-6, 0.25])
def test_gateconv_forward_magnitude_matches_numpy(eps):
    H, k, v, _, wh, wv, cw = _gc_case()
    res = oracle.gateconv_fwd_f64(H, k, v, wh, wv, cw, eps=eps, mags=True, threads=2)
    ref = np_gateconv_fwd_mag(H, k, v, wh, wv, cw, eps)
    np.testing.assert_allclose(res[6], ref, rtol=1e-11, atol=0)
    assert np.all(res[6] >= np.abs(res[0]) * (1 - RT))


def test_gateconv_backward_magnitudes_match_numpy():
    H, k, v, dY, wh, wv, cw = _gc_case()
    _, vhat, al, rh, rk, rv = oracle.gateconv_fwd_f64(H, k, v, wh, wv, cw, threads=2)
    res = oracle.gateconv_bwd_f64(dY, H, k, v, wh, wv, cw, vhat, al, rh, rk, rv, mags=True, threads=2)
    ref = np_gateconv_bwd_mags(dY, H, k, v, wh, wv, cw, vhat, al, rh, rk, rv)
    for name, got, want in zip(("magH", "magk", "magv", "mdwh", "mdwv", "mdcw"), res[6:], ref):
        np.testing.assert_allclose(got, want, rtol=1e-11, atol=0, err_msg=name)
    for val, mag in zip(res[:6], res[6:]):
        assert np.all(mag >= np.abs(val) * (1 - 1e-9))
