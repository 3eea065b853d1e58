"""Pins of the fp64 oracle to what the pages and the mathematics fix.

Every test here runs on the CPU.  The oracle is checked against closed forms,
invariants stated by the "Engram saved-state gate" page (masking, the packed
grad_kv value sum), special cases, and fp64 central differences of its own
forward (so a dropped term, wrong sign or transposed index in the backward
fails).  No expected value here comes from the oracle itself.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import synth
from numerics import bf16_to_f64, f32_to_bf16_bits

EPS = float(np.float32(1e-20))
CLAMP = float(np.float32(1e-6))
D = 5120


def sigmoid(z):
    return 1.0 / (1.0 + math.exp(-z))


def inputs(n, d=D, seed=0, p=1.0, grad=True):
    return synth.host_inputs(n, seed=seed, p=p, d=d, grad=grad)


# --------------------------------------------------------------------------
# bf16 rounding, by the IEEE-754 / bfloat16 bit definition
# --------------------------------------------------------------------------

@pytest.mark.parametrize("val,bits", [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),                 # exact tie, even neighbour below
    (1.0 + 3 * 2.0 ** -8, 0x3F82),             # exact tie, odd below -> round up
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),    # just above the tie
    (-0.0, 0x8000),
    (float("inf"), 0x7F80),
    (float(np.finfo(np.float32).max), 0x7F80),  # rounds up to +inf
    (2.0 ** -133, 0x0001),                     # smallest bf16 subnormal
    (-2.5, 0xC020),
])
def test_bf16_rne_definition(val, bits):
    f = np.float32(val)
    assert oracle.f32_to_bf16(float(f)) == bits
    assert int(f32_to_bf16_bits(np.array([f]))[0]) == bits


def test_bf16_nan_stays_quiet_nan():
    b = oracle.f32_to_bf16(float("nan"))
    assert (b & 0x7F80) == 0x7F80 and (b & 0x007F) != 0


# --------------------------------------------------------------------------
# masking: a masked token's output is its X row, bit for bit (semantics paragraph)
# --------------------------------------------------------------------------

def test_mask_false_output_is_x_bitwise_and_gradients_vanish():
    n = 6
    inp = inputs(n, seed=11)
    x, kv, w, g = inp["x"].copy(), inp["kv"], inp["weight"], inp["grad_out"]
    x[1, 2, :7] = 0x8000  # negative zeros survive only through a bit copy
    mask = np.array([1, 0, 1, 0, 0, 1], np.uint8)
    out, saved = oracle.fwd_bf16(x, kv, w, mask)
    out_all, saved_all = oracle.fwd_bf16(x, kv, w, np.ones(n, np.uint8))
    off = mask == 0
    assert np.array_equal(out[off], x[off])
    assert np.all(saved[off][:, :, 0] == 0.0)
    # dot and both rstd are the true values for masked tokens (reading R7)
    assert np.array_equal(saved[off][:, :, 1:], saved_all[off][:, :, 1:])
    assert not np.array_equal(out[~off], x[~off])

    dx, dkv, dw = oracle.bwd_bf16(x, kv, w, saved, g)
    assert np.array_equal(dx[off], g[off])  # dx = G exactly (G is already bf16)
    assert np.all(bf16_to_f64(dkv[off]) == 0.0)
    # grad_weight gets nothing from masked tokens
    _, _, dw_masked_only = oracle.bwd_bf16(x[off], kv[off], w, saved[off], g[off])
    assert np.all(dw_masked_only == 0.0)


# --------------------------------------------------------------------------
# zero rows: dot == 0 exactly, sgn(0) = 0 -> gate 1/2 (reading R1)
# --------------------------------------------------------------------------

def test_zero_x_row_gives_half_gate_and_exact_half_value():
    inp = inputs(2, seed=12)
    x, kv, w, g = inp["x"].copy(), inp["kv"].copy(), inp["weight"], inp["grad_out"]
    x[0, 1, :] = 0
    kv[1, 2 * D:3 * D] = 0
    mask = np.ones(2, np.uint8)
    out, saved = oracle.fwd_bf16(x, kv, w, mask)
    for (t, s) in [(0, 1), (1, 2)]:
        assert saved[t, s, 1] == 0.0
        assert saved[t, s, 0] == 0.5
    # rstd of a zero row is (eps)^(-1/2) rounded to fp32
    assert saved[0, 1, 2] == np.float32(1.0 / math.sqrt(EPS))
    assert saved[1, 2, 3] == np.float32(1.0 / math.sqrt(EPS))
    # zero X row: out = v / 2, which is exact in bf16 (power-of-two scale)
    v0 = bf16_to_f64(kv[0, 4 * D:])
    assert np.array_equal(bf16_to_f64(out[0, 1]), v0 / 2)

    dx, dkv, dw = oracle.bwd_bf16(x, kv, w, saved, g)
    assert np.array_equal(dx[0, 1], g[0, 1])
    assert np.all(bf16_to_f64(dkv[0, D:2 * D]) == 0.0)
    assert np.array_equal(dx[1, 2], g[1, 2])
    assert np.all(bf16_to_f64(dkv[1, 2 * D:3 * D]) == 0.0)


# --------------------------------------------------------------------------
# clamp: |dot| < 1e-6 -> z = sgn(dot) sqrt(1e-6), zero derivative (R2)
# --------------------------------------------------------------------------

def test_clamp_rows():
    n = 4
    inp = inputs(n, seed=13)
    x, kv, w, g = inp["x"], inp["kv"].copy(), inp["weight"], inp["grad_out"]
    # scale every key row by 2^-64 (exact in bf16: only the exponent moves)
    keys = kv[:, :4 * D]
    nz = (keys & 0x7F80) != 0
    keys[nz] = keys[nz] - np.uint16(64 << 7)
    kv[:, :4 * D] = keys
    mask = np.ones(n, np.uint8)
    out, saved, out64, saved64, aux = oracle.fwd_bf16(x, kv, w, mask, extras=True)
    dots = saved64[:, :, 1]
    assert np.all(np.abs(dots) < CLAMP) and np.all(dots != 0.0)
    for t in range(n):
        for s in range(4):
            want = sigmoid(math.copysign(math.sqrt(CLAMP), dots[t, s]))
            assert abs(saved64[t, s, 0] - want) <= 1e-15
            assert aux[t, s, 1] == 0.0
    dx, dkv, dw = oracle.bwd_bf16(x, kv, w, saved, g)
    assert np.array_equal(dx, g)
    assert np.all(bf16_to_f64(dkv[:, :4 * D]) == 0.0)
    assert np.all(dw == 0.0)
    # the value gradient still flows through the clamped gate
    assert np.any(bf16_to_f64(dkv[:, 4 * D:]) != 0.0)


def test_clamp_boundary_passes_gradient_at_equality():
    # one stream, d = 1: x = k = 1 gives rstd = (1 + eps)^(-1/2) = 1 in fp64,
    # so dot = w exactly; w = c sits on the boundary, w = c*(1-2^-30) below it.
    d = 1
    x = np.ones((1, 4, d))
    kv = np.ones((1, 5 * d))
    g = np.ones((1, 4, d))
    for wv, passes in [(CLAMP, True), (CLAMP * (1 - 2.0 ** -30), False)]:
        w = np.full((4, d), wv)
        out, saved = oracle.fwd_f64(x, kv, w, np.ones(1, np.uint8))
        assert saved[0, 0, 1] == wv
        dx, dkv, dw = oracle.bwd_f64(x, kv, w, saved, g)
        gate = saved[0, 0, 0]
        # dL/dw = delta * x^ k^ = delta;  delta = dg g(1-g) / (2 sqrt c) or 0
        want = gate * (1 - gate) / (2 * math.sqrt(wv)) if passes else 0.0
        assert dw[0, 0] == pytest.approx(want, rel=1e-14, abs=0.0)


# --------------------------------------------------------------------------
# constant rows: rstd = (1 + eps)^(-1/2), dot = sum_j w_j
# --------------------------------------------------------------------------

def test_constant_rows():
    inp = inputs(1, seed=14)
    w = inp["weight"]
    x = np.full((1, 4, D), 0x3F80, np.uint16)   # 1.0
    kv = np.full((1, 5 * D), 0x3F80, np.uint16)
    out, saved, out64, saved64, aux = oracle.fwd_bf16(x, kv, w, np.ones(1, np.uint8), extras=True)
    for s in range(4):
        assert saved64[0, s, 2] == 1.0 / math.sqrt(1.0 + EPS)
        assert saved64[0, s, 3] == 1.0 / math.sqrt(1.0 + EPS)
        exact = math.fsum(float(v) for v in w[s])
        assert abs(saved64[0, s, 1] - exact) <= 1e-12 * abs(exact)
        assert saved64[0, s, 0] == pytest.approx(sigmoid(math.sqrt(exact)), rel=1e-14)


# --------------------------------------------------------------------------
# a four-stream closed-form token (d = 4), derived by hand
# --------------------------------------------------------------------------

def test_closed_form_tiny_token():
    d = 4
    # stream 0: x = k = (1,1,1,1) -> rstd = 1 (fp64: 1 + 1e-20 == 1); w sums to 1 -> dot 1
    # stream 1: x = (2,0,0,0), k = (-2,0,0,0) -> mean square 1, rstd 1; dot = -4 w0 = -1
    # stream 2: x = k = (1,1,1,1), w = 1/2 each -> dot 2
    # stream 3: x = (1,-1,1,-1), k = (1,1,1,1), w = 1 -> dot 0 -> gate 1/2
    x = np.array([[[1, 1, 1, 1], [2, 0, 0, 0], [1, 1, 1, 1], [1, -1, 1, -1]]], float)
    keys = np.array([[1, 1, 1, 1], [-2, 0, 0, 0], [1, 1, 1, 1], [1, 1, 1, 1]], float)
    v = np.array([2.0, -1.0, 0.5, 0.0])
    kv = np.concatenate([keys.ravel(), v])[None, :]
    w = np.array([[0.5, 0.25, 0.125, 0.125], [0.25, 1, 1, 1], [0.5] * 4, [1.0] * 4])
    G = np.array([[[1, 0, 0, 0], [0, 1, 0, 0], [0, 0, 0, 0], [1, 1, 1, 1]]], float)
    out, saved = oracle.fwd_f64(x, kv, w, np.ones(1, np.uint8))
    s1, sm1, s2 = sigmoid(1.0), sigmoid(-1.0), sigmoid(math.sqrt(2.0))
    gates = [s1, sm1, s2, 0.5]
    dots = [1.0, -1.0, 2.0, 0.0]
    for s in range(4):
        assert saved[0, s, 1] == pytest.approx(dots[s], rel=1e-15, abs=1e-300)
        assert saved[0, s, 0] == pytest.approx(gates[s], rel=1e-15)
        assert saved[0, s, 2] == 1.0 and saved[0, s, 3] == 1.0
        np.testing.assert_allclose(out[0, s], x[0, s] + gates[s] * v, rtol=1e-15, atol=1e-15)

    dx, dkv, dw = oracle.bwd_f64(x, kv, w, saved, G)
    # stream 0: dg = G.v = 2; delta = 2 s1 (1-s1) / (2 sqrt 1) = s1 sm1
    #   dx_j = G_j + delta (w_j k^_j - dot x^_j / 4) = G_j + delta (w_j - 1/4)
    #   dk_j = delta (w_j x^_j - dot k^_j / 4) = delta (w_j - 1/4);  dw_j = delta
    d0 = s1 * sm1
    np.testing.assert_allclose(dx[0, 0], [1 + d0 * 0.25, 0, -0.125 * d0, -0.125 * d0], rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(dkv[0, 0:4], [0.25 * d0, 0, -0.125 * d0, -0.125 * d0], rtol=1e-14, atol=1e-16)
    np.testing.assert_allclose(dw[0], [d0] * 4, rtol=1e-14)
    # stream 1: dg = G.v = -1; dz = -sm1 (1 - sm1) = -sm1 s1; delta = dz / 2
    #   x^ = (2,0,0,0), k^ = (-2,0,0,0), dot = -1
    #   dx_0 = 0 + delta (w0 k^0 - dot x^0 / 4) = delta (0.25*-2 + 2/4) = 0; dx_1 = G_1 = 1
    #   dk_0 = delta (w0 x^0 - dot k^0 / 4) = delta (0.5 - 0.5) = 0
    #   dw_0 = delta x^0 k^0 = -4 delta
    d1 = -sm1 * s1 / 2
    np.testing.assert_allclose(dx[0, 1], [0, 1, 0, 0], atol=1e-16)
    np.testing.assert_allclose(dkv[0, 4:8], [0, 0, 0, 0], atol=1e-16)
    np.testing.assert_allclose(dw[1], [-4 * d1, 0, 0, 0], rtol=1e-14, atol=1e-300)
    # stream 2: G = 0 -> no gradient at all
    assert np.all(dx[0, 2] == 0) and np.all(dkv[0, 8:12] == 0) and np.all(dw[2] == 0)
    # stream 3: dot = 0 < c -> delta = 0: dx = G, dk = 0, dw = 0
    np.testing.assert_array_equal(dx[0, 3], G[0, 3])
    assert np.all(dkv[0, 12:16] == 0) and np.all(dw[3] == 0)
    # shared value: dv = sum_s gate_s G_s
    want_dv = s1 * G[0, 0] + sm1 * G[0, 1] + s2 * G[0, 2] + 0.5 * G[0, 3]
    np.testing.assert_allclose(dkv[0, 16:20], want_dv, rtol=1e-15)


# --------------------------------------------------------------------------
# invariances
# --------------------------------------------------------------------------

def _f64_inputs(n, d, seed):
    inp = inputs(n, d=d, seed=seed)
    return (bf16_to_f64(inp["x"]), bf16_to_f64(inp["kv"]), inp["weight"].astype(np.float64),
            bf16_to_f64(inp["grad_out"]))


def test_power_of_two_scaling():
    x, kv, w, _ = _f64_inputs(2, D, 15)
    mask = np.ones(2, np.uint8)
    _, base = oracle.fwd_f64(x, kv, w, mask)
    x2 = x.copy(); x2[0, 1] *= 8.0
    kv2 = kv.copy(); kv2[1, 3 * D:4 * D] *= 2.0 ** -5
    _, sc = oracle.fwd_f64(x2, kv2, w, mask)
    assert sc[0, 1, 1] == pytest.approx(base[0, 1, 1], rel=1e-12)
    assert sc[0, 1, 0] == pytest.approx(base[0, 1, 0], rel=1e-12)
    assert sc[0, 1, 2] == pytest.approx(base[0, 1, 2] / 8.0, rel=1e-12)
    assert sc[1, 3, 1] == pytest.approx(base[1, 3, 1], rel=1e-12)
    assert sc[1, 3, 3] == pytest.approx(base[1, 3, 3] * 32.0, rel=1e-12)
    untouched = np.ones((2, 4), bool); untouched[0, 1] = untouched[1, 3] = False
    assert np.array_equal(sc[untouched], base[untouched])


def test_key_negation_flips_dot_and_gate():
    x, kv, w, _ = _f64_inputs(3, D, 16)
    mask = np.ones(3, np.uint8)
    _, base = oracle.fwd_f64(x, kv, w, mask)
    kv2 = kv.copy(); kv2[:, :4 * D] *= -1.0
    _, neg = oracle.fwd_f64(x, kv2, w, mask)
    assert np.array_equal(neg[:, :, 1], -base[:, :, 1])
    np.testing.assert_allclose(neg[:, :, 0], 1.0 - base[:, :, 0], rtol=0, atol=1e-15)


def test_stream_permutation_permutes_everything():
    n = 3
    x, kv, w, g = _f64_inputs(n, D, 17)
    mask = np.array([1, 1, 0], np.uint8)
    perm = [2, 0, 3, 1]
    kp = kv[:, :4 * D].reshape(n, 4, D)[:, perm].reshape(n, 4 * D)
    kvp = np.concatenate([kp, kv[:, 4 * D:]], axis=1)
    out, sv = oracle.fwd_f64(x, kv, w, mask)
    outp, svp = oracle.fwd_f64(x[:, perm], kvp, w[perm], mask)
    assert np.array_equal(outp, out[:, perm])
    assert np.array_equal(svp, sv[:, perm])
    dx, dkv, dw = oracle.bwd_f64(x, kv, w, sv, g)
    dxp, dkvp, dwp = oracle.bwd_f64(x[:, perm], kvp, w[perm], svp, g[:, perm])
    assert np.array_equal(dxp, dx[:, perm])
    assert np.array_equal(dkvp[:, :4 * D].reshape(n, 4, D), dkv[:, :4 * D].reshape(n, 4, D)[:, perm])
    assert np.array_equal(dwp, dw[perm])
    # the shared-value gradient sums streams in another order: equal up to rounding
    np.testing.assert_allclose(dkvp[:, 4 * D:], dkv[:, 4 * D:], rtol=1e-14, atol=1e-14)


def test_value_gradient_is_sum_of_stream_contributions():
    """Layout paragraph: grad of the shared value sums the four stream terms before the cast."""
    n = 4
    inp = inputs(n, seed=18)
    x, kv, w, g = inp["x"], inp["kv"], inp["weight"], inp["grad_out"]
    out, saved = oracle.fwd_bf16(x, kv, w, np.ones(n, np.uint8))
    gates = saved[:, :, 0].astype(np.float64)
    G = bf16_to_f64(g)
    _, dkv, _, _, dkv64, _, _, _, _ = oracle.bwd_bf16(x, kv, w, saved, g, extras=True)
    want = np.zeros((n, D))
    for s in range(4):
        want += gates[:, s:s + 1] * G[:, s]
    np.testing.assert_allclose(dkv64[:, 4 * D:], want, rtol=1e-15, atol=1e-300)
    # a single nonzero stream: dv = bf16(gate_s * G_s) with one rounding chain
    g1 = np.zeros_like(g); g1[:, 2] = g[:, 2]
    _, dkv1, _ = oracle.bwd_bf16(x, kv, w, saved, g1)
    single = (gates[:, 2:3] * G[:, 2]).astype(np.float32)
    assert np.array_equal(dkv1[:, 4 * D:], f32_to_bf16_bits(single))
    # summing before the cast differs from casting each contribution and adding
    per_stream = sum(bf16_to_f64(f32_to_bf16_bits((gates[:, s:s + 1] * G[:, s]).astype(np.float32)))
                     for s in range(4))
    assert not np.array_equal(bf16_to_f64(dkv[:, 4 * D:]), per_stream)


def test_thread_count_does_not_change_results():
    n = 37
    inp = inputs(n, seed=19, p=0.7)
    x, kv, w, m, g = inp["x"], inp["kv"], inp["weight"], inp["mask"], inp["grad_out"]
    o1, s1 = oracle.fwd_bf16(x, kv, w, m, threads=1)
    o5, s5 = oracle.fwd_bf16(x, kv, w, m, threads=5)
    assert np.array_equal(o1, o5) and np.array_equal(s1, s5)
    a = oracle.bwd_bf16(x, kv, w, s1, g, threads=1, extras=True)
    b = oracle.bwd_bf16(x, kv, w, s1, g, threads=5, extras=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    np.testing.assert_allclose(a[5], b[5], rtol=1e-13, atol=1e-13)


def test_rounded_outputs_are_rounded_fp64_views():
    n = 5
    inp = inputs(n, seed=20, p=0.6)
    out, saved, out64, saved64, aux = oracle.fwd_bf16(inp["x"], inp["kv"], inp["weight"], inp["mask"],
                                                      extras=True)
    on = inp["mask"] != 0
    assert np.array_equal(out[on], f32_to_bf16_bits(out64[on].astype(np.float32)))
    assert np.array_equal(saved, saved64.astype(np.float32))


# --------------------------------------------------------------------------
# backward == gradient of the forward (fp64 central differences)
# --------------------------------------------------------------------------

def _loss(x, kv, w, mask, G):
    out, _ = oracle.fwd_f64(x, kv, w, mask)
    return float(np.sum(G * out))


def _fd_setup(n, d, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 4, d))
    kv = rng.standard_normal((n, 5 * d))
    w = 1.0 + 0.1 * rng.standard_normal((4, d))
    G = rng.standard_normal((n, 4, d))
    mask = np.ones(n, np.uint8)
    mask[-1] = 0
    _, sv = oracle.fwd_f64(x, kv, w, mask)
    # keep every row away from the clamp band and the sign kink
    assert np.all(np.abs(sv[:, :, 1]) > 1e-2)
    return x, kv, w, mask, G, sv


def test_backward_matches_central_differences_every_coordinate_d16():
    n, d, h = 3, 16, 1e-6
    x, kv, w, mask, G, sv = _fd_setup(n, d, 21)
    dx, dkv, dw = oracle.bwd_f64(x, kv, w, sv, G)
    for name, arr, grad in (("x", x, dx), ("kv", kv, dkv), ("w", w, dw)):
        flat = arr.reshape(-1)
        for i in range(flat.size):
            keep = flat[i]
            flat[i] = keep + h
            lp = _loss(x, kv, w, mask, G)
            flat[i] = keep - h
            lm = _loss(x, kv, w, mask, G)
            flat[i] = keep
            fd = (lp - lm) / (2 * h)
            an = grad.reshape(-1)[i]
            assert abs(fd - an) <= 1e-5 * max(abs(an), 1e-2), (name, i, fd, an)


def test_backward_matches_central_differences_d5120():
    n, d, h = 2, D, 1e-6
    x, kv, w, mask, G, sv = _fd_setup(n, d, 22)
    dx, dkv, dw = oracle.bwd_f64(x, kv, w, sv, G)
    rng = np.random.default_rng(23)
    for name, arr, grad in (("x", x, dx), ("kv", kv, dkv), ("w", w, dw)):
        flat = arr.reshape(-1)
        gflat = grad.reshape(-1)
        base = flat.copy()
        # random directions
        for _ in range(6):
            u = rng.standard_normal(flat.size)
            u /= np.linalg.norm(u)
            flat[:] = base + h * u
            lp = _loss(x, kv, w, mask, G)
            flat[:] = base - h * u
            lm = _loss(x, kv, w, mask, G)
            flat[:] = base
            fd = (lp - lm) / (2 * h)
            an = float(gflat @ u)
            assert abs(fd - an) <= 1e-5 * max(abs(an), 1e-2), (name, "dir", fd, an)
        # sampled coordinates, including key, value and masked-token columns
        for i in rng.choice(flat.size, 24, replace=False):
            flat[i] = base[i] + h
            lp = _loss(x, kv, w, mask, G)
            flat[i] = base[i] - h
            lm = _loss(x, kv, w, mask, G)
            flat[i] = base[i]
            fd = (lp - lm) / (2 * h)
            assert abs(fd - gflat[i]) <= 1e-5 * max(abs(gflat[i]), 1e-2), (name, int(i), fd, gflat[i])


# --------------------------------------------------------------------------
# fused weight = wh * we and its product rule
# --------------------------------------------------------------------------

def test_fused_weight_is_the_exact_product():
    """bf16 x bf16 has at most 16 significant bits: exact in fp32."""
    from fractions import Fraction
    wh = synth.normal_bf16(4 * 64, 3, 21).reshape(4, 64)
    we = synth.normal_bf16(4 * 64, 3, 22).reshape(4, 64)
    got = oracle.fused_weight(wh, we)
    a, b = bf16_to_f64(wh).ravel(), bf16_to_f64(we).ravel()
    for i in range(a.size):
        assert Fraction(float(got.ravel()[i])) == Fraction(a[i]) * Fraction(b[i])


def test_product_rule_matches_central_differences():
    """dL/dwh and dL/dwe through weight = wh * we, against fp64 differences of
    the forward evaluated with the composed weight."""
    n, d, h = 2, 8, 1e-6
    rng = np.random.default_rng(31)
    x = rng.standard_normal((n, 4, d))
    kv = rng.standard_normal((n, 5 * d))
    G = rng.standard_normal((n, 4, d))
    mask = np.ones(n, np.uint8)
    wh16 = f32_to_bf16_bits((1.0 + 0.1 * rng.standard_normal((4, d))).astype(np.float32))
    we16 = f32_to_bf16_bits((1.0 + 0.1 * rng.standard_normal((4, d))).astype(np.float32))
    wh, we = bf16_to_f64(wh16), bf16_to_f64(we16)
    w = wh * we
    _, sv = oracle.fwd_f64(x, kv, w, mask)
    assert np.all(np.abs(sv[:, :, 1]) > 1e-2)
    _, _, dw = oracle.bwd_f64(x, kv, w, sv, G)
    gwh, gwe = oracle.weight_grads(dw, wh16, we16)

    def loss(a, b):
        out, _ = oracle.fwd_f64(x, kv, a * b, mask)
        return float(np.sum(G * out))

    for (s_, j) in [(0, 0), (1, 3), (3, 7), (2, 5)]:
        e = np.zeros((4, d)); e[s_, j] = h
        fd_h = (loss(wh + e, we) - loss(wh - e, we)) / (2 * h)
        fd_e = (loss(wh, we + e) - loss(wh, we - e)) / (2 * h)
        assert abs(fd_h - gwh[s_, j]) <= 1e-5 * max(abs(gwh[s_, j]), 1e-2)
        assert abs(fd_e - gwe[s_, j]) <= 1e-5 * max(abs(gwe[s_, j]), 1e-2)
