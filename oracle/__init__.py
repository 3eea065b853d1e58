"""fp64 CPU oracle for the four-stream Engram saved-state gate.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``.  The product library never loads it.

The arithmetic lives in ``engram_oracle.c`` (plain C, fp64); this module only
builds it with gcc when no built copy exists and marshals numpy arrays.
Which page passage each step follows is stated in the C file's header.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "engram_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libengram_oracle.so")

D_MODEL = 5120  # per-stream hidden size of the gate as specified
N_STREAMS = 4


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call([
            "gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
            "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm", "-lpthread",
        ])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None
# ENGRAM_ORACLE_LIB names another build of engram_oracle.c; the mutation tests
# set it to check that the pins reject planted mistakes.
_lib_path_override = os.environ.get("ENGRAM_ORACLE_LIB") or None


def use_library(path):
    """Load the oracle from another build of engram_oracle.c (the mutation
    tests use this to check that the pins reject planted mistakes)."""
    global _lib, _lib_path_override
    _lib = None
    _lib_path_override = path


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(_lib_path_override or build())
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.engram_oracle_fwd_f64.argtypes = [I64, I64, P, P, P, P, P, P, P, ctypes.c_int]
        lib.engram_oracle_bwd_f64.argtypes = [I64, I64, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_int]
        lib.engram_oracle_fwd_bf16.argtypes = [I64, I64, P, P, P, P, P, P, P, P, P, ctypes.c_int]
        lib.engram_oracle_bwd_bf16.argtypes = [I64, I64, P, P, P, P, P, P, P, P, P, P, P, P, P, P,
                                               ctypes.c_int]
        for f in (lib.engram_oracle_fwd_f64, lib.engram_oracle_bwd_f64,
                  lib.engram_oracle_fwd_bf16, lib.engram_oracle_bwd_bf16):
            f.restype = ctypes.c_int
        lib.engram_oracle_fused_weight.argtypes = [I64, P, P, P]
        lib.engram_oracle_fused_weight.restype = ctypes.c_int
        lib.engram_oracle_weight_grads.argtypes = [I64, P, P, P, P, P]
        lib.engram_oracle_weight_grads.restype = ctypes.c_int
        lib.engram_oracle_gateconv_fwd_f64.argtypes = [I64, I64, I64, ctypes.c_double] + [P] * 13 + [ctypes.c_int]
        lib.engram_oracle_gateconv_fwd_f64.restype = ctypes.c_int
        lib.engram_oracle_gateconv_bwd_f64.argtypes = [I64, I64, I64] + [P] * 24 + [ctypes.c_int]
        lib.engram_oracle_gateconv_bwd_f64.restype = ctypes.c_int
        lib.engram_oracle_round_bf16.argtypes = [I64, P, P]
        lib.engram_oracle_round_bf16.restype = ctypes.c_int
        lib.engram_oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        lib.engram_oracle_f32_to_bf16.restype = ctypes.c_uint16
        _lib = lib
    return _lib


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def _arr(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def fwd_f64(x, kv, w, mask, threads: int = 1, aux: bool = False):
    """fp64 forward, no rounding.  Shapes: x [n,4,d], kv [n,5d], w [4,d], mask [n].

    Returns (out [n,4,d], saved [n,4,4]) or, with aux=True, also aux [n,4,2]
    = (sum |x^ w k^|, d gate / d dot).
    """
    x = _arr(x, np.float64)
    kv = _arr(kv, np.float64)
    w = _arr(w, np.float64)
    mask = _arr(mask, np.uint8)
    n, s, d = x.shape
    assert s == N_STREAMS and kv.shape == (n, 5 * d) and w.shape == (N_STREAMS, d)
    out = np.empty_like(x)
    saved = np.empty((n, N_STREAMS, 4), np.float64)
    ax = np.empty((n, N_STREAMS, 2), np.float64) if aux else None
    rc = _load().engram_oracle_fwd_f64(d, n, _ptr(x), _ptr(kv), _ptr(w), _ptr(mask), _ptr(out),
                                       _ptr(saved), _ptr(ax), threads)
    if rc != 0:
        raise RuntimeError(f"oracle fwd_f64 failed: {rc}")
    return (out, saved, ax) if aux else (out, saved)


def bwd_f64(x, kv, w, saved, g, threads: int = 1, mags: bool = False):
    """fp64 backward from an fp64 saved state.  Returns (dx, dkv, dw) [+ mags]."""
    x = _arr(x, np.float64)
    kv = _arr(kv, np.float64)
    w = _arr(w, np.float64)
    saved = _arr(saved, np.float64)
    g = _arr(g, np.float64)
    n, s, d = x.shape
    dx = np.empty_like(x)
    dkv = np.empty((n, 5 * d), np.float64)
    dw = np.empty((N_STREAMS, d), np.float64)
    m = (np.empty_like(dx), np.empty_like(dkv), np.empty_like(dw)) if mags else (None, None, None)
    rc = _load().engram_oracle_bwd_f64(d, n, _ptr(x), _ptr(kv), _ptr(w), _ptr(saved), _ptr(g),
                                       _ptr(dx), _ptr(dkv), _ptr(dw), _ptr(m[0]), _ptr(m[1]),
                                       _ptr(m[2]), threads)
    if rc != 0:
        raise RuntimeError(f"oracle bwd_f64 failed: {rc}")
    return (dx, dkv, dw) + (m if mags else ())


def fwd_bf16(x16, kv16, w32, mask, threads: int = 1, extras: bool = False):
    """Forward on storage types.

    x16 [n,4,d] uint16 (bf16 bits), kv16 [n,5d] uint16, w32 [4,d] float32,
    mask [n] uint8.  Returns (out16 uint16 [n,4,d], saved float32 [n,4,4]);
    with extras=True also (out64, saved64, aux) in fp64.
    """
    x16 = _arr(x16, np.uint16)
    kv16 = _arr(kv16, np.uint16)
    w32 = _arr(w32, np.float32)
    mask = _arr(mask, np.uint8)
    n, s, d = x16.shape
    assert s == N_STREAMS and kv16.shape == (n, 5 * d) and w32.shape == (N_STREAMS, d)
    out = np.empty_like(x16)
    saved = np.empty((n, N_STREAMS, 4), np.float32)
    if extras:
        out64 = np.empty(x16.shape, np.float64)
        saved64 = np.empty((n, N_STREAMS, 4), np.float64)
        aux = np.empty((n, N_STREAMS, 2), np.float64)
    else:
        out64 = saved64 = aux = None
    rc = _load().engram_oracle_fwd_bf16(d, n, _ptr(x16), _ptr(kv16), _ptr(w32), _ptr(mask),
                                        _ptr(out), _ptr(saved), _ptr(out64), _ptr(saved64),
                                        _ptr(aux), threads)
    if rc != 0:
        raise RuntimeError(f"oracle fwd_bf16 failed: {rc}")
    return (out, saved, out64, saved64, aux) if extras else (out, saved)


def bwd_bf16(x16, kv16, w32, saved32, g16, threads: int = 1, extras: bool = False):
    """Backward on storage types from a given fp32 saved state.

    Returns (dx16, dkv16, dw32); with extras=True also
    (dx64, dkv64, dw64, mag_dx, mag_dkv, mag_dw).
    """
    x16 = _arr(x16, np.uint16)
    kv16 = _arr(kv16, np.uint16)
    w32 = _arr(w32, np.float32)
    saved32 = _arr(saved32, np.float32)
    g16 = _arr(g16, np.uint16)
    n, s, d = x16.shape
    dx = np.empty_like(x16)
    dkv = np.empty((n, 5 * d), np.uint16)
    dw = np.empty((N_STREAMS, d), np.float32)
    if extras:
        ex = (np.empty(x16.shape, np.float64), np.empty((n, 5 * d), np.float64),
              np.empty((N_STREAMS, d), np.float64), np.empty(x16.shape, np.float64),
              np.empty((n, 5 * d), np.float64), np.empty((N_STREAMS, d), np.float64))
    else:
        ex = (None,) * 6
    rc = _load().engram_oracle_bwd_bf16(d, n, _ptr(x16), _ptr(kv16), _ptr(w32), _ptr(saved32),
                                        _ptr(g16), _ptr(dx), _ptr(dkv), _ptr(dw),
                                        *[_ptr(e) for e in ex], threads)
    if rc != 0:
        raise RuntimeError(f"oracle bwd_bf16 failed: {rc}")
    return (dx, dkv, dw) + (ex if extras else ())


def f32_to_bf16(f: float) -> int:
    return int(_load().engram_oracle_f32_to_bf16(ctypes.c_float(f)))


def fused_weight(wh16, we16):
    """weight fp32 = fp32(wh) * fp32(we) for bf16-bit arrays of equal shape."""
    wh16 = _arr(wh16, np.uint16)
    we16 = _arr(we16, np.uint16)
    assert wh16.shape == we16.shape
    out = np.empty(wh16.shape, np.float32)
    rc = _load().engram_oracle_fused_weight(wh16.size, _ptr(wh16), _ptr(we16), _ptr(out))
    if rc != 0:
        raise RuntimeError(f"oracle fused_weight failed: {rc}")
    return out


def weight_grads(dw64, wh16, we16):
    """Product rule of weight = wh * we: returns (grad_wh, grad_we) in fp64."""
    dw64 = _arr(dw64, np.float64)
    wh16 = _arr(wh16, np.uint16)
    we16 = _arr(we16, np.uint16)
    gwh = np.empty(dw64.shape, np.float64)
    gwe = np.empty(dw64.shape, np.float64)
    rc = _load().engram_oracle_weight_grads(dw64.size, _ptr(dw64), _ptr(wh16), _ptr(we16), _ptr(gwh), _ptr(gwe))
    if rc != 0:
        raise RuntimeError(f"oracle weight_grads failed: {rc}")
    return gwh, gwe


# ---------------- Engram GateConv (TileOPs "Engram Operators" page) ----------------

GATECONV_TAPS = 4


def round_bf16(x64):
    """fp64 -> fp32 (RNE) -> bf16 (RNE) bits."""
    x64 = _arr(x64, np.float64)
    out = np.empty(x64.shape, np.uint16)
    rc = _load().engram_oracle_round_bf16(x64.size, _ptr(x64), _ptr(out))
    if rc != 0:
        raise RuntimeError("oracle round_bf16 failed")
    return out


def gateconv_fwd_f64(H, k, v, wh, wv, cw, eps=1e-6, mags=False, threads=None):
    """GateConv forward in fp64.  H, k, v [M,T,d]; wh, wv [d]; cw [4,d].

    Returns (Y, vhat, alpha, rrms_h, rrms_k, rrms_v) [+ magY].
    """
    H, k, v = (_arr(a, np.float64) for a in (H, k, v))
    wh, wv, cw = (_arr(a, np.float64) for a in (wh, wv, cw))
    M, T, d = H.shape
    assert k.shape == v.shape == H.shape and wh.shape == wv.shape == (d,) and cw.shape == (GATECONV_TAPS, d)
    Y, vhat = np.empty_like(H), np.empty_like(H)
    al, rh, rk, rv = (np.empty((M, T), np.float64) for _ in range(4))
    mY = np.empty_like(H) if mags else None
    rc = _load().engram_oracle_gateconv_fwd_f64(M, T, d, eps, _ptr(H), _ptr(k), _ptr(v), _ptr(wh), _ptr(wv),
                                                _ptr(cw), _ptr(Y), _ptr(vhat), _ptr(al), _ptr(rh), _ptr(rk),
                                                _ptr(rv), _ptr(mY), threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle gateconv_fwd_f64 failed: {rc}")
    return (Y, vhat, al, rh, rk, rv) + ((mY,) if mags else ())


def gateconv_bwd_f64(dY, H, k, v, wh, wv, cw, vhat, alpha, rrh, rrk, rrv, mags=False, threads=None):
    """GateConv backward in fp64 from the saved tensors.

    Returns (dH, dk, dv, dwh, dwv, dcw) [+ (magH, magk, magv, mdwh, mdwv, mdcw)].
    """
    dY, H, k, v, vhat = (_arr(a, np.float64) for a in (dY, H, k, v, vhat))
    wh, wv, cw = (_arr(a, np.float64) for a in (wh, wv, cw))
    alpha, rrh, rrk, rrv = (_arr(a, np.float64) for a in (alpha, rrh, rrk, rrv))
    M, T, d = H.shape
    dH, dk, dv = np.empty_like(H), np.empty_like(H), np.empty_like(H)
    dwh, dwv, dcw = np.empty(d), np.empty(d), np.empty((GATECONV_TAPS, d))
    m = ((np.empty_like(H), np.empty_like(H), np.empty_like(H), np.empty(d), np.empty(d),
          np.empty((GATECONV_TAPS, d))) if mags else (None,) * 6)
    rc = _load().engram_oracle_gateconv_bwd_f64(M, T, d, _ptr(dY), _ptr(H), _ptr(k), _ptr(v), _ptr(wh), _ptr(wv),
                                                _ptr(cw), _ptr(vhat), _ptr(alpha), _ptr(rrh), _ptr(rrk), _ptr(rrv),
                                                _ptr(dH), _ptr(dk), _ptr(dv), _ptr(dwh), _ptr(dwv), _ptr(dcw),
                                                *[_ptr(x) for x in m], threads or default_threads())
    if rc != 0:
        raise RuntimeError(f"oracle gateconv_bwd_f64 failed: {rc}")
    return (dH, dk, dv, dwh, dwv, dcw) + (m if mags else ())
