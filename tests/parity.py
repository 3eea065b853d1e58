"""Element-by-element comparison of device results with the fp64 oracle.

Bars (from the fp32 evaluation error of each quantity, bounded by a multiple
of the unit roundoff times the magnitude of its terms, plus the bf16 store):
  forward  rstd_X, rstd_key  rel 1e-5
           dot               1e-5 |dot| + 2^-22 A,  A = sum_j |x^ w k^|
           gate              1e-5 g + |dg/ddot| tol_dot;  exactly 0 when masked
           out               within 1 bf16 ulp of the unrounded fp64 value, widened
                             by |v| tol_gate + 32 u32 (|x| + |g v|); masked tokens
                             must be bit copies of X
  backward (fed the oracle's fp32 saved, so both sides start from the same state)
           grad_x, grad_kv   within 1 bf16 ulp of the unrounded value, widened by
                             32 u32 (magnitude scale from the oracle, which bounds
                             delta through sum |G v|); norm-wise rel L2 against the
                             oracle's rounded bf16 values <= 2e-3
           grad_weight       1e-3 |ref| + 1e-4 + 2^-20 C,  C = sum_t |delta| x^ k^|
                             with |delta| bounded through sum |G v| as above.
                             The worst-case rounding bound of the device's
                             summation (about 120 sequential fp32 roundings per
                             element: the grad-of-gate reduction inside delta,
                             32 tokens per wave, the slot combine, then the
                             partial-row reduction) is ~2^-17 C; the bar uses
                             the tighter 2^-20 C, which the rounding errors,
                             being independent, stay far below (the largest
                             |error| / C seen is reported as dw_err_over_C).
"""
from __future__ import annotations

import numpy as np

import oracle
from numerics import U32, bf16_to_f64, check_bf16, check_rel

D = 5120
CHUNK = 256  # tokens per comparison chunk (bounds host memory)


def _rel_l2(got, ref):
    got = np.asarray(got, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got))


class _Agg:
    """Accumulates chunked check_bf16 statistics."""

    def __init__(self):
        self.n = self.eq = 0
        self.dr = self.rr = self.d64 = self.r64 = 0.0

    def add(self, r):
        self.n += r["n"]
        self.eq += r["bit_equal_to_rounded_oracle"]
        self.dr += r["sq_diff_rounded"]
        self.rr += r["sq_rounded"]
        self.d64 += r["sq_diff_fp64"]
        self.r64 += r["sq_fp64"]

    def report(self, st, key):
        st[f"{key}_bit_equal_frac"] = self.eq / max(self.n, 1)
        # norm-wise error against the oracle's rounded bf16 values (the gate)
        st[f"{key}_rel_l2"] = float(np.sqrt(self.dr / self.rr)) if self.rr > 0 else float(np.sqrt(self.dr))
        # and against its unrounded fp64 values (includes bf16 storage rounding)
        st[f"{key}_rel_l2_fp64"] = float(np.sqrt(self.d64 / self.r64)) if self.r64 > 0 else 0.0


def check_fwd(inp, out16, saved32, threads=8, ref=None):
    """Compare a device forward with the oracle on the same input bytes."""
    x, kv, w, mask = inp["x"], inp["kv"], inp["weight"], inp["mask"]
    if ref is None:
        ref = oracle.fwd_bf16(x, kv, w, mask, threads=threads, extras=True)
    out_ref, saved_ref, out64, saved64, aux = ref
    on = mask != 0
    st = {"tokens": int(mask.size), "masked": int((~on).sum())}

    # masked tokens: bit copy of X, gate saved as 0 (reading R7)
    assert np.array_equal(out16[~on], x[~on]), "masked token output is not a bit copy of X"
    assert np.all(saved32[~on][:, :, 0] == 0.0), "masked token saved a nonzero gate"

    st["rstd_x_maxrel"] = check_rel("rstd_X", saved32[..., 2], saved64[..., 2], 1e-5)
    st["rstd_k_maxrel"] = check_rel("rstd_key", saved32[..., 3], saved64[..., 3], 1e-5)
    tol_dot = 1e-5 * np.abs(saved64[..., 1]) + 2.0 ** -22 * aux[..., 0]
    check_rel("dot", saved32[..., 1], saved64[..., 1], 0.0, atol=tol_dot)
    st["dot_maxrel"] = float(np.max(np.abs(saved32[..., 1] - saved64[..., 1]) /
                                    np.maximum(np.abs(saved64[..., 1]), 1e-30)))
    tol_g = 1e-5 * np.abs(saved64[..., 0]) + aux[..., 1] * tol_dot
    check_rel("gate", saved32[..., 0], saved64[..., 0], 0.0, atol=tol_g)
    st["gate_maxrel_vs_spec"] = float(np.max(np.abs(saved32[..., 0] - saved64[..., 0]) /
                                             np.maximum(np.abs(saved64[..., 0]), 1e-30)))

    agg = _Agg()
    idx = np.nonzero(on)[0]
    for c0 in range(0, idx.size, CHUNK):
        sel = idx[c0:c0 + CHUNK]
        xs = bf16_to_f64(x[sel])                           # [m,4,d]
        vs = bf16_to_f64(kv[sel][:, 4 * D:])[:, None, :]   # [m,1,d]
        g = saved64[sel][:, :, 0:1]
        mag = np.abs(xs) + np.abs(g * vs)
        extra = np.abs(vs) * tol_g[sel][:, :, None]
        agg.add(check_bf16("out", out16[sel], out64[sel], mag, extra=extra))
    if agg.n:
        agg.report(st, "out")
    return st


def check_bwd(inp, saved32, dx16, dkv16, dw32, threads=8, ref=None):
    """Compare a device backward with the oracle; both consume `saved32`."""
    x, kv, w, g = inp["x"], inp["kv"], inp["weight"], inp["grad_out"]
    if ref is None:
        ref = oracle.bwd_bf16(x, kv, w, saved32, g, threads=threads, extras=True)
    dx_r, dkv_r, dw_r, dx64, dkv64, dw64, mdx, mdkv, mdw = ref
    st = {}
    for name, key, got, r64, mag in (("grad_x", "dx", dx16, dx64, mdx), ("grad_kv", "dkv", dkv16, dkv64, mdkv)):
        agg = _Agg()
        for c0 in range(0, got.shape[0], CHUNK):
            sl = slice(c0, c0 + CHUNK)
            agg.add(check_bf16(name, got[sl], r64[sl], mag[sl]))
        agg.report(st, key)
    st["dw_maxrel"] = check_rel("grad_weight", dw32, dw64, 1e-3, atol=1e-4 + 2.0 ** -20 * mdw)
    err = np.abs(dw32.astype(np.float64) - dw64)
    st["dw_err_over_C"] = float(np.max(err / np.maximum(mdw, 1e-300)))
    # elements outside a plain rel 1e-3 / abs 1e-4 bar (allowed by the C term where the sum cancels)
    st["dw_outside_rel1e-3_abs1e-4"] = int(np.count_nonzero(err > 1e-3 * np.abs(dw64) + 1e-4))
    st["dw_rel_l2"] = _rel_l2(dw32, dw64)
    for k in ("dx_rel_l2", "dkv_rel_l2", "dw_rel_l2"):
        assert st[k] <= 2e-3, f"{k} = {st[k]:.3e} exceeds 2e-3"
    return st


def check_bwd_end_to_end(inp, saved_dev, dx16, dkv16, dw32, fwd_ref, threads=8):
    """Device backward on the device's own saved vs the oracle backward on the
    oracle's saved.

    delta = dg g(1-g) / (2 sqrt|dot|) has |d ln(delta) / d dot| <=
    |1 - 2g| / (2 sqrt|dot|) + 1 / (2 |dot|), so the forward's admissible dot
    error (1e-5 |dot| + 2^-22 A) can move delta by a large relative amount on
    rows with |dot| near that noise floor.  grad_x and grad_key are therefore
    gated norm-wise (<= 2e-3) on rows whose propagated delta error is <= 1e-3;
    grad_value (which depends on the gates only) on all rows; grad_weight, a
    sum over all rows, is reported.
    """
    x, kv, w, g = inp["x"], inp["kv"], inp["weight"], inp["grad_out"]
    saved_ref, saved64, aux = fwd_ref[1], fwd_ref[3], fwd_ref[4]
    dx_r, dkv_r, dw_r = oracle.bwd_bf16(x, kv, w, saved_ref, g, threads=threads)
    n = x.shape[0]
    dot = np.abs(saved64[..., 1])
    gate = saved64[..., 0]
    tol_dot = 1e-5 * dot + 2.0 ** -22 * aux[..., 0]
    with np.errstate(divide="ignore", invalid="ignore"):
        sens = np.abs(1 - 2 * gate) / (2 * np.sqrt(dot)) + 1 / (2 * dot)
        rel_delta = np.where(dot > 0, sens * tol_dot, np.inf)
    ok = rel_delta <= 1e-3                                   # [n, 4]
    gx, rx_ = bf16_to_f64(dx16), bf16_to_f64(dx_r)
    gk = bf16_to_f64(dkv16[:, :4 * D]).reshape(n, 4, D)
    rk_ = bf16_to_f64(dkv_r[:, :4 * D]).reshape(n, 4, D)
    st = {"e2e_rows_excluded": int((~ok).sum()),
          "e2e_dx_rel_l2": _rel_l2(gx[ok], rx_[ok]),
          "e2e_dk_rel_l2": _rel_l2(gk[ok], rk_[ok]),
          "e2e_dv_rel_l2": _rel_l2(bf16_to_f64(dkv16[:, 4 * D:]), bf16_to_f64(dkv_r[:, 4 * D:])),
          "e2e_dx_rel_l2_all_rows": _rel_l2(gx, rx_),
          "e2e_dw_rel_l2_reported": _rel_l2(dw32, dw_r)}
    for k in ("e2e_dx_rel_l2", "e2e_dk_rel_l2", "e2e_dv_rel_l2"):
        assert st[k] <= 2e-3, f"{k} = {st[k]:.3e} exceeds 2e-3"
    return st
