"""Pins of the fp64 GateConv oracle (TileOPs "Engram Operators" page, GateConv
section) to closed forms, structural invariants the page states (causal,
depthwise, per-sequence) and fp64 central differences of the forward.
None of the expected values comes from the oracle itself."""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle

EPS = 1e-6


def sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def rand_case(M, T, d, seed):
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((M, T, d))
    k = rng.standard_normal((M, T, d))
    v = rng.standard_normal((M, T, d))
    wh = 1.0 + 0.2 * rng.standard_normal(d)
    wv = 1.0 + 0.2 * rng.standard_normal(d)
    cw = 0.5 * rng.standard_normal((4, d))
    return H, k, v, wh, wv, cw


def test_alpha_closed_forms():
    M, T, d = 1, 3, 16
    H, k, v, wh, wv, cw = rand_case(M, T, d, 1)
    k[0, 0] = 0.0                      # <h^, k^> = 0 -> alpha = 1/2
    k[0, 1] = H[0, 1]                  # k = H, w_h = 1 -> s = d r^2 mean(H^2) / sqrt(d)
    wh = np.ones(d)
    Y, vhat, al, rh, rk, rv = oracle.gateconv_fwd_f64(H, k, v, wh, wv, cw)
    assert al[0, 0] == 0.5
    ms = np.mean(H[0, 1] ** 2)
    s = d * ms / (ms + EPS) / math.sqrt(d)
    assert al[0, 1] == pytest.approx(1 / (1 + math.exp(-s)), rel=1e-14)
    assert rh[0, 1] == pytest.approx(1 / math.sqrt(ms + EPS), rel=1e-14)


def test_rrms_v_closed_form_and_vhat():
    M, T, d = 1, 2, 8
    H, k, v, wh, wv, cw = rand_case(M, T, d, 2)
    v[0, 0] = 3.0  # constant row: vhat = 3 alpha, rrms_v = (9 alpha^2 + eps)^(-1/2)
    Y, vhat, al, rh, rk, rv = oracle.gateconv_fwd_f64(H, k, v, wh, wv, cw)
    a = al[0, 0]
    np.testing.assert_allclose(vhat[0, 0], 3 * a, rtol=1e-15)
    assert rv[0, 0] == pytest.approx(1 / math.sqrt(9 * a * a + EPS), rel=1e-14)
    np.testing.assert_allclose(vhat[0, 1], al[0, 1] * v[0, 1], rtol=1e-15)


def test_identity_tap_gives_pointwise_map():
    """conv_w = (0, 0, 0, 1): c_t = u_t, so Y_t = SiLU(vhat rrms_v w_v) + vhat."""
    M, T, d = 2, 5, 12
    H, k, v, wh, wv, cw = rand_case(M, T, d, 3)
    cw = np.zeros((4, d)); cw[3] = 1.0
    Y, vhat, al, rh, rk, rv = oracle.gateconv_fwd_f64(H, k, v, wh, wv, cw)
    u = vhat * rv[..., None] * wv
    np.testing.assert_allclose(Y, u * sigmoid(u) + vhat, rtol=1e-14, atol=1e-15)


def test_single_tap_delays_by_three_tokens():
    """conv_w = (1, 0, 0, 0): c_t = u_{t-3}; the first three tokens see zero history."""
    M, T, d = 1, 7, 8
    H, k, v, wh, wv, cw = rand_case(M, T, d, 4)
    cw = np.zeros((4, d)); cw[0] = 1.0
    Y, vhat, al, rh, rk, rv = oracle.gateconv_fwd_f64(H, k, v, wh, wv, cw)
    u = vhat * rv[..., None] * wv
    np.testing.assert_allclose(Y[0, :3], vhat[0, :3], rtol=0, atol=0)  # SiLU(0) = 0
    c = u[0, :-3]
    np.testing.assert_allclose(Y[0, 3:], c * sigmoid(c) + vhat[0, 3:], rtol=1e-14, atol=1e-15)


def test_causal_and_sequence_independent():
    M, T, d = 3, 9, 8
    H, k, v, wh, wv, cw = rand_case(M, T, d, 5)
    base = oracle.gateconv_fwd_f64(H, k, v, wh, wv, cw)[0]
    for t in (0, 4, 8):
        H2, v2 = H.copy(), v.copy()
        H2[1, t] += 0.3
        v2[1, t] -= 0.7
        Y2 = oracle.gateconv_fwd_f64(H2, k, v2, wh, wv, cw)[0]
        assert np.array_equal(Y2[1, :t], base[1, :t])          # no effect on the past
        assert np.array_equal(Y2[[0, 2]], base[[0, 2]])        # no effect on other sequences
        assert not np.array_equal(Y2[1, t], base[1, t])


def test_zero_history_equals_zero_value_tokens():
    """Three leading tokens with v = 0 contribute u = 0, which is what the
    causal zero padding assumes before t = 0 (reading G5)."""
    M, T, d = 1, 6, 8
    H, k, v, wh, wv, cw = rand_case(M, T, d, 6)
    rng = np.random.default_rng(7)
    pre = rng.standard_normal((1, 3, d))
    Hp = np.concatenate([pre, H], axis=1)
    kp = np.concatenate([pre, k], axis=1)
    vp = np.concatenate([np.zeros((1, 3, d)), v], axis=1)
    Y = oracle.gateconv_fwd_f64(H, k, v, wh, wv, cw)[0]
    Yp = oracle.gateconv_fwd_f64(Hp, kp, vp, wh, wv, cw)[0]
    np.testing.assert_allclose(Yp[:, 3:], Y, rtol=1e-14, atol=1e-15)


def _loss(dY, H, k, v, wh, wv, cw):
    return float(np.sum(dY * oracle.gateconv_fwd_f64(H, k, v, wh, wv, cw)[0]))


def test_backward_matches_central_differences_every_coordinate():
    M, T, d, h = 2, 6, 8, 1e-6
    H, k, v, wh, wv, cw = rand_case(M, T, d, 8)
    dY = np.random.default_rng(9).standard_normal((M, T, d))
    Y, vhat, al, rh, rk, rv = oracle.gateconv_fwd_f64(H, k, v, wh, wv, cw)
    grads = oracle.gateconv_bwd_f64(dY, H, k, v, wh, wv, cw, vhat, al, rh, rk, rv)
    names = ("H", "k", "v", "wh", "wv", "cw")
    arrs = [H, k, v, wh, wv, cw]
    for name, arr, g in zip(names, arrs, grads):
        flat = arr.reshape(-1)
        for i in range(flat.size):
            keep = flat[i]
            flat[i] = keep + h
            lp = _loss(dY, *arrs)
            flat[i] = keep - h
            lm = _loss(dY, *arrs)
            flat[i] = keep
            fd = (lp - lm) / (2 * h)
            an = g.reshape(-1)[i]
            assert abs(fd - an) <= 1e-5 * max(abs(an), 1e-2), (name, i, fd, an)


def test_backward_directional_at_width_5120():
    M, T, d, h = 1, 5, 5120, 1e-6
    H, k, v, wh, wv, cw = rand_case(M, T, d, 10)
    dY = np.random.default_rng(11).standard_normal((M, T, d))
    Y, vhat, al, rh, rk, rv = oracle.gateconv_fwd_f64(H, k, v, wh, wv, cw)
    grads = oracle.gateconv_bwd_f64(dY, H, k, v, wh, wv, cw, vhat, al, rh, rk, rv)
    arrs = [H, k, v, wh, wv, cw]
    rng = np.random.default_rng(12)
    for arr, g in zip(arrs, grads):
        flat = arr.reshape(-1)
        base = flat.copy()
        for _ in range(3):
            u = rng.standard_normal(flat.size)
            u /= np.linalg.norm(u)
            flat[:] = base + h * u
            lp = _loss(dY, *arrs)
            flat[:] = base - h * u
            lm = _loss(dY, *arrs)
            flat[:] = base
            fd = (lp - lm) / (2 * h)
            an = float(g.reshape(-1) @ u)
            assert abs(fd - an) <= 1e-5 * max(abs(an), 1e-2), (fd, an)


def test_magnitudes_bound_the_values():
    M, T, d = 2, 7, 16
    H, k, v, wh, wv, cw = rand_case(M, T, d, 13)
    dY = np.random.default_rng(14).standard_normal((M, T, d))
    Y, vhat, al, rh, rk, rv, mY = oracle.gateconv_fwd_f64(H, k, v, wh, wv, cw, mags=True)
    assert np.all(mY >= np.abs(Y) * (1 - 1e-12))
    out = oracle.gateconv_bwd_f64(dY, H, k, v, wh, wv, cw, vhat, al, rh, rk, rv, mags=True)
    for val, mag in zip(out[:6], out[6:]):
        assert np.all(mag >= np.abs(val) * (1 - 1e-12))
