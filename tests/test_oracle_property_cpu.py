"""Invariances of the gate's definition, checked on the fp64 oracle over random
sizes, inputs, masks, scales and stream orders (hypothesis).

The relations follow from the definition ("Engram saved-state gate",
semantics paragraph) alone, so none of the expected values comes from the
oracle: a wrong index, sign or transposed operand that the fixed-case pins
happen to miss shows up on some random case.
  - mask false: out = X, saved gate 0, grad_x = G, no key, value or weight
    gradient from that token;
  - X row times 2^a, key row times 2^b: dot and gate unchanged, rstd_X and
    rstd_key times 2^-a and 2^-b, grad_key times 2^-b, grad_weight unchanged;
  - all keys negated: dot negated, gate -> 1 - gate, both rstd unchanged,
    grad_key unchanged, grad_weight negated;
  - streams permuted (X, grad_out, key blocks, weight rows): every output
    permuted alike; the shared value's gradient unchanged up to the order of
    its four-term sum.  Checked on the fp64 path and on the storage-type path
    (bf16 in and out, fp32 saved state), where it holds bit for bit but for
    the value gradient's last bf16 rounding;
  - Euler's relation: the gate does not change when a stream's X row or key
    row is scaled, so the gate's share of grad_x (grad_x - G) is orthogonal
    to X, and grad_key is orthogonal to its key row, per (token, stream).
eps = 1e-20 is below half an fp64 ulp of these rows' mean squares, so the
scale relations hold to rounding.
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

import oracle  # noqa: E402

PERMS = list(itertools.permutations(range(4)))


@st.composite
def _case(draw):
    n = draw(st.integers(1, 5))
    d = draw(st.sampled_from([4, 8, 16, 40, 64]))
    seed = draw(st.integers(0, 2 ** 31 - 1))
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 4, d))
    kv = rng.standard_normal((n, 5 * d))
    w = 1.0 + 0.1 * rng.standard_normal((4, d))
    g = rng.standard_normal((n, 4, d))
    mask = (rng.random(n) < 0.7).astype(np.uint8)
    return n, d, x, kv, w, g, mask


def _run(x, kv, w, g, mask):
    out, sv = oracle.fwd_f64(x, kv, w, mask)
    dx, dkv, dw = oracle.bwd_f64(x, kv, w, sv, g)
    return out, sv, dx, dkv, dw


def _bf16(a):
    """fp64 values to bf16 bit patterns (ties to even; normal values)."""
    u = np.asarray(a, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _close(a, b, rel):
    scale = max(np.max(np.abs(b)), 1e-300)
    assert np.max(np.abs(a - b)) <= rel * scale


@settings(max_examples=60, deadline=None)
@given(_case())
def test_masked_tokens(case):
    n, d, x, kv, w, g, mask = case
    out, sv, dx, dkv, dw = _run(x, kv, w, g, mask)
    off = mask == 0
    assert np.array_equal(out[off], x[off])
    assert np.all(sv[off, :, 0] == 0.0)
    assert np.array_equal(dx[off], g[off])
    assert np.all(dkv[off] == 0.0)
    # grad_weight gets nothing from masked tokens: dropping them changes nothing
    on = ~off
    if on.any():
        _, svo = oracle.fwd_f64(x[on], kv[on], w, mask[on])
        _close(oracle.bwd_f64(x[on], kv[on], w, svo, g[on])[2], dw, 1e-13)
    else:
        assert np.all(dw == 0.0)


@settings(max_examples=60, deadline=None)
@given(_case(), st.integers(-6, 6), st.integers(-6, 6))
def test_power_of_two_scales(case, a, b):
    n, d, x, kv, w, g, mask = case
    out, sv, dx, dkv, dw = _run(x, kv, w, g, mask)
    kv2 = kv.copy()
    kv2[:, :4 * d] *= 2.0 ** b
    out2, sv2, dx2, dkv2, dw2 = _run(x * 2.0 ** a, kv2, w, g, mask)
    _close(sv2[..., 0], sv[..., 0], 1e-12)                   # gate
    _close(sv2[..., 1], sv[..., 1], 1e-12)                   # dot
    _close(sv2[..., 2], sv[..., 2] * 2.0 ** -a, 1e-12)       # rstd_X
    _close(sv2[..., 3], sv[..., 3] * 2.0 ** -b, 1e-12)       # rstd_key
    _close(dkv2[:, :4 * d], dkv[:, :4 * d] * 2.0 ** -b, 1e-10)
    _close(dkv2[:, 4 * d:], dkv[:, 4 * d:], 1e-12)           # grad_value: gate and G only
    _close(dw2, dw, 1e-10)


@settings(max_examples=60, deadline=None)
@given(_case())
def test_key_negation(case):
    n, d, x, kv, w, g, mask = case
    out, sv, dx, dkv, dw = _run(x, kv, w, g, mask)
    kv2 = kv.copy()
    kv2[:, :4 * d] *= -1.0
    out2, sv2, dx2, dkv2, dw2 = _run(x, kv2, w, g, mask)
    assert np.array_equal(sv2[..., 1], -sv[..., 1])
    assert np.array_equal(sv2[..., 2], sv[..., 2]) and np.array_equal(sv2[..., 3], sv[..., 3])
    on = mask.astype(bool)
    np.testing.assert_allclose(sv2[on, :, 0], 1.0 - sv[on, :, 0], rtol=0, atol=1e-15)
    _close(dkv2[:, :4 * d], dkv[:, :4 * d], 1e-9)
    _close(dw2, -dw, 1e-9)


@settings(max_examples=60, deadline=None)
@given(_case(), st.sampled_from(PERMS))
def test_stream_permutation(case, perm):
    n, d, x, kv, w, g, mask = case
    perm = list(perm)
    out, sv, dx, dkv, dw = _run(x, kv, w, g, mask)
    kp = kv[:, :4 * d].reshape(n, 4, d)[:, perm].reshape(n, 4 * d)
    kvp = np.concatenate([kp, kv[:, 4 * d:]], axis=1)
    outp, svp, dxp, dkvp, dwp = _run(x[:, perm], kvp, w[perm], g[:, perm], mask)
    assert np.array_equal(outp, out[:, perm])
    assert np.array_equal(svp, sv[:, perm])
    assert np.array_equal(dxp, dx[:, perm])
    assert np.array_equal(dkvp[:, :4 * d].reshape(n, 4, d), dkv[:, :4 * d].reshape(n, 4, d)[:, perm])
    assert np.array_equal(dwp, dw[perm])
    _close(dkvp[:, 4 * d:], dkv[:, 4 * d:], 1e-14)


@settings(max_examples=60, deadline=None)
@given(_case())
def test_euler_orthogonality(case):
    n, d, x, kv, w, g, mask = case
    out, sv, dx, dkv, dw = _run(x, kv, w, g, mask)
    gate_x = dx - g                                   # the gate's share of grad_x
    dk = dkv[:, :4 * d].reshape(n, 4, d)
    k = kv[:, :4 * d].reshape(n, 4, d)
    # grad_x is stored as G plus the gate's share, so taking G back out carries
    # the rounding of |G|: the bound counts it
    for share, row, carried in ((gate_x, x, g), (dk, k, 0.0)):
        dots = np.sum(share * row, axis=2)
        mags = np.sum(np.abs(row) * (np.abs(share) + np.abs(carried)), axis=2)
        assert np.all(np.abs(dots) <= 1e-11 * mags + 1e-300), np.max(np.abs(dots) / np.maximum(mags, 1e-300))
    # and the relation is not empty: unmasked tokens do move grad_x and grad_key
    on = mask.astype(bool)
    if on.any():
        assert np.any(gate_x[on] != 0.0) and np.any(dk[on] != 0.0)


@settings(max_examples=40, deadline=None)
@given(_case(), st.sampled_from(PERMS))
def test_stream_permutation_storage_types(case, perm):
    n, d, x, kv, w, g, mask = case
    perm = list(perm)
    x16, kv16, g16, w32 = _bf16(x), _bf16(kv), _bf16(g), w.astype(np.float32)
    out, sv = oracle.fwd_bf16(x16, kv16, w32, mask)
    dx, dkv, dw = oracle.bwd_bf16(x16, kv16, w32, sv, g16)
    kp = kv16[:, :4 * d].reshape(n, 4, d)[:, perm].reshape(n, 4 * d)
    kvp = np.ascontiguousarray(np.concatenate([kp, kv16[:, 4 * d:]], axis=1))
    xp, gp = np.ascontiguousarray(x16[:, perm]), np.ascontiguousarray(g16[:, perm])
    outp, svp = oracle.fwd_bf16(xp, kvp, np.ascontiguousarray(w32[perm]), mask)
    dxp, dkvp, dwp = oracle.bwd_bf16(xp, kvp, np.ascontiguousarray(w32[perm]), svp, gp)
    assert np.array_equal(outp, out[:, perm])
    assert np.array_equal(svp.view(np.uint32), sv[:, perm].view(np.uint32))
    assert np.array_equal(dxp, dx[:, perm])
    assert np.array_equal(dkvp[:, :4 * d].reshape(n, 4, d), dkv[:, :4 * d].reshape(n, 4, d)[:, perm])
    assert np.array_equal(dwp.view(np.uint32), dw[perm].view(np.uint32))
    # the value gradient: a reordered fp64 four-term sum, then one bf16 rounding
    # (one bf16 ulp apart at most; absolute near zero, where the sign may flip)
    va = (dkv[:, 4 * d:].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    vb = (dkvp[:, 4 * d:].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    bound = 2.0 ** -7 * np.maximum(np.abs(va), np.abs(vb)) + 1e-14 * max(np.max(np.abs(va)), 1e-300)
    assert np.all(np.abs(va - vb) <= bound)
