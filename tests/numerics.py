"""Storage-type helpers and comparison rules shared by the tests.

Comparison rules (each derived from the fp32 arithmetic of the kernels: a
value computed in fp32 differs from its exact value by at most a small
multiple of the fp32 unit roundoff times the sum of the magnitudes of the
terms that formed it, and the bf16 store adds one rounding):

* bf16 outputs: the device value must lie within one bf16 ulp of the oracle's
  unrounded fp64 value, widened by an fp32-evaluation allowance
  ``err = kappa * 2^-24 * mag`` where ``mag`` is the oracle's sum of |terms|
  of that element (plus any propagated scalar tolerance).
* fp32 scalars: relative 1e-5, plus a conditioning term where the value is a
  cancelling sum (the dot).
"""
from __future__ import annotations

import numpy as np

U32 = 2.0 ** -24  # fp32 unit roundoff


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 (bit definition; NaN kept quiet)."""
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return r


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (8 significant bits)."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    a = np.maximum(a, 2.0 ** -126)
    e = np.floor(np.log2(a))
    return np.ldexp(1.0, (e - 7).astype(np.int64))


def check_bf16(name, got_bits, ref64, mag, kappa=32.0, extra=None, max_report=5):
    """Assert |got - ref| <= ulp_bf16(|ref| + err) + err elementwise.

    err = kappa * 2^-24 * mag (+ extra).  Returns a dict of statistics.
    """
    got = bf16_to_f64(got_bits).ravel()
    ref = np.asarray(ref64, dtype=np.float64).ravel()
    err = kappa * U32 * np.asarray(mag, dtype=np.float64).ravel()
    if extra is not None:
        err = err + np.asarray(extra, dtype=np.float64).ravel()
    tol = ulp_bf16(np.abs(ref) + err) + err
    diff = np.abs(got - ref)
    bad = ~(diff <= tol)
    # identical bit patterns always pass (covers inf/nan copies)
    if bad.any():
        idx = np.nonzero(bad)[0][:max_report]
        detail = ", ".join(f"[{i}] got={got[i]!r} ref={ref[i]!r} tol={tol[i]:.3g}" for i in idx)
        raise AssertionError(f"{name}: {int(bad.sum())}/{bad.size} elements outside 1 bf16 ulp: {detail}")
    ref_bits = f32_to_bf16_bits(ref.astype(np.float32))
    exact = np.count_nonzero(np.asarray(got_bits).ravel() == ref_bits)
    ref_r = bf16_to_f64(ref_bits)
    return {"n": int(ref.size), "bit_equal_to_rounded_oracle": int(exact),
            # squared norms for norm-wise errors (aggregated over chunks by the caller)
            "sq_diff_rounded": float(np.sum((got - ref_r) ** 2)), "sq_rounded": float(np.sum(ref_r ** 2)),
            "sq_diff_fp64": float(np.sum((got - ref) ** 2)), "sq_fp64": float(np.sum(ref ** 2))}


def check_rel(name, got, ref, rtol, atol=None, max_report=5):
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    tol = rtol * np.abs(ref)
    if atol is not None:
        tol = tol + np.asarray(atol, dtype=np.float64).ravel()
    diff = np.abs(got - ref)
    bad = ~(diff <= tol)
    if bad.any():
        idx = np.nonzero(bad)[0][:max_report]
        detail = ", ".join(f"[{i}] got={got[i]!r} ref={ref[i]!r} tol={tol[i]:.3g}" for i in idx)
        raise AssertionError(f"{name}: {int(bad.sum())}/{bad.size} outside tolerance: {detail}")
    return float(np.max(diff / np.maximum(np.abs(ref), 1e-300))) if ref.size else 0.0


def subnormal_bf16(bits):
    """bf16 bits with the exponent cleared (sign and mantissa kept, never zero):
    subnormal values in [2^-133, 2^-126)."""
    return ((bits & 0x8000) | ((bits & 0x007F) | 0x0001)).astype(np.uint16)


def subnormal_rows_case(n=256, seed=7):
    """The backward's subnormal case: tokens 0-31 with subnormal grad_out rows,
    32-63 with subnormal value rows, 64-95 both, the rest normal; mask all ones."""
    import synth
    inp = synth.host_inputs(n, seed=seed, p=1.0, grad=True)
    g, kv = inp["grad_out"], inp["kv"]
    g[0:32] = subnormal_bf16(g[0:32])
    kv[32:64, 4 * 5120:] = subnormal_bf16(kv[32:64, 4 * 5120:])
    g[64:96] = subnormal_bf16(g[64:96])
    kv[64:96, 4 * 5120:] = subnormal_bf16(kv[64:96, 4 * 5120:])
    return inp
