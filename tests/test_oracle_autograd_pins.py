"""Pins of the oracle's backward against automatic differentiation.

The oracle's backward formulas are derived by hand.  Here each forward is
written out from its definition in plain PyTorch fp64 (CPU), torch.autograd
differentiates the scalar L = sum(grad_out * output), and the oracle's
backward (fed the oracle's own fp64 forward state) must agree with autograd
at every coordinate to ~1e-11: a dropped term, a wrong sign or a transposed
operand in any gradient fails here whatever the forward does.

Gate ("Engram saved-state gate", semantics paragraph), per token and stream:
  x^ = x (mean x^2 + eps)^-1/2, k^ likewise, dot = sum x^ w k^,
  gate = sigmoid(sgn(dot) sqrt(max(|dot|, c))), out = mask ? x + gate v : x,
with eps and c the FP32 constants 1e-20f and 1e-6f of an FP32 computation,
widened exactly (the library's reading R3).
GateConv ("Engram Operators", GateConv section; readings G1-G6 of this
library): h^ = H rrms_h w_h, k^ = k rrms_k w_h, alpha = sigmoid(<h^, k^> /
sqrt(d)), vhat = alpha v, u = vhat rrms_v w_v, c_t = sum_i conv_w[i] u_{t-3+i}
(causal within each sequence), Y = SiLU(c) + vhat.  For GateConv this pins the
backward to those readings, not the readings to the page.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle

RTOL = 1e-11
EPS = float(np.float32(1e-20))
CLAMP = float(np.float32(1e-6))


def _close(name, got, want):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    scale = np.max(np.abs(want)) + 1e-300
    err = np.max(np.abs(got - want)) / scale
    assert err <= RTOL, f"{name}: max |oracle - autograd| / max |autograd| = {err:.3e}"


def _gate_forward_torch(x, kv, w, mask):
    n, S, d = x.shape
    k = kv[:, : S * d].reshape(n, S, d)
    v = kv[:, S * d:]
    rx = (x.pow(2).mean(-1, keepdim=True) + EPS).rsqrt()
    rk = (k.pow(2).mean(-1, keepdim=True) + EPS).rsqrt()
    dot = ((x * rx) * w[None] * (k * rk)).sum(-1)
    z = torch.sign(dot) * torch.sqrt(torch.clamp(dot.abs(), min=CLAMP))
    gate = torch.sigmoid(z)
    out = torch.where(mask[:, None, None], x + gate[..., None] * v[:, None, :], x)
    return out, dot, rx[..., 0], rk[..., 0]


@pytest.mark.parametrize("d,seed", [(16, 0), (40, 1)])
def test_gate_backward_matches_autograd(d, seed):
    rng = np.random.default_rng(seed)
    n = 7
    x = rng.standard_normal((n, 4, d))
    kv = rng.standard_normal((n, 5 * d))
    w = 1.0 + 0.1 * rng.standard_normal((4, d))
    g = rng.standard_normal((n, 4, d))
    mask = np.ones(n, np.uint8)
    mask[2] = 0                    # a masked token
    kv[4, 1 * d:2 * d] = 0.0       # a zero key row: dot = 0, the clamp path, sgn(0) = 0
    x[5, 2] = 0.0                  # a zero X row: rstd_X = eps^-1/2, dot = 0
    out_o, saved = oracle.fwd_f64(x, kv, w, mask)
    dx, dkv, dw = oracle.bwd_f64(x, kv, w, saved, g)

    tx, tkv, tw = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (x, kv, w))
    out, dot, rx, rk = _gate_forward_torch(tx, tkv, tw, torch.tensor(mask.astype(bool)))
    _close("out (the forward itself)", out_o, out.detach().numpy())
    _close("saved dot", saved[..., 1], dot.detach().numpy())
    _close("saved rstd_X", saved[..., 2], rx.detach().numpy())
    _close("saved rstd_key", saved[..., 3], rk.detach().numpy())
    (out * torch.tensor(g)).sum().backward()
    _close("grad_x", dx, tx.grad.numpy())
    _close("grad_kv", dkv, tkv.grad.numpy())
    _close("grad_weight", dw, tw.grad.numpy())
    # the cases are what they claim
    assert saved[4, 1, 1] == 0.0 and saved[5, 2, 1] == 0.0 and saved[2, :, 0].tolist() == [0.0] * 4


def _gateconv_forward_torch(H, k, v, wh, wv, cw, eps=1e-6):
    M, T, d = H.shape
    rrh = (H.pow(2).mean(-1, keepdim=True) + eps).rsqrt()
    rrk = (k.pow(2).mean(-1, keepdim=True) + eps).rsqrt()
    hh = H * rrh * wh
    kh = k * rrk * wh
    alpha = torch.sigmoid((hh * kh).sum(-1, keepdim=True) / np.sqrt(d))
    vhat = alpha * v
    rrv = (vhat.pow(2).mean(-1, keepdim=True) + eps).rsqrt()
    u = vhat * rrv * wv
    taps = cw.shape[0]
    upad = torch.cat([torch.zeros(M, taps - 1, d, dtype=u.dtype), u], dim=1)  # zero history per sequence
    c = sum(cw[i] * upad[:, i:i + T] for i in range(taps))
    return torch.nn.functional.silu(c) + vhat


@pytest.mark.parametrize("M,T,d,seed", [(2, 7, 16, 3), (1, 11, 24, 4)])
def test_gateconv_backward_matches_autograd(M, T, d, seed):
    rng = np.random.default_rng(seed)
    H, k, v, dY = (rng.standard_normal((M, T, d)) for _ in range(4))
    wh = 1.0 + 0.25 * rng.standard_normal(d)
    wv = 1.0 + 0.25 * rng.standard_normal(d)
    cw = 0.5 * rng.standard_normal((4, d))
    Y, vhat, al, rh, rk, rv = oracle.gateconv_fwd_f64(H, k, v, wh, wv, cw, threads=1)
    dH, dk, dv, dwh, dwv, dcw = oracle.gateconv_bwd_f64(dY, H, k, v, wh, wv, cw, vhat, al, rh, rk, rv, threads=1)

    t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (H, k, v, wh, wv, cw)]
    out = _gateconv_forward_torch(*t)
    _close("Y (the forward itself)", Y, out.detach().numpy())
    (out * torch.tensor(dY)).sum().backward()
    for name, got, tt in (("dH", dH, t[0]), ("dk", dk, t[1]), ("dv", dv, t[2]), ("drms_w_h", dwh, t[3]),
                          ("drms_w_v", dwv, t[4]), ("dconv_w", dcw, t[5])):
        _close(name, got, tt.grad.numpy())
