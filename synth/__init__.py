"""Seeded, counter-based synthetic inputs for the Engram gate workloads.

Shared by the tests (both the oracle side and the HIP side) and by
``bench.py``.  It holds input generation only -- none of the gate's
arithmetic.  The recipe (SplitMix64 words, 12-field Irwin-Hall normals,
24-bit Bernoulli masks, edge rows) is documented in ``synth_host.c``; the
device twin ``synth_dev.hip`` produces the same bytes on the GPU.

Tensor ids: X = 1, KV = 2, weight = 3, mask = 4, grad_out = 5,
edge-row selection = 6, zero-row selection = 7.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_HOST_SRC = os.path.join(_HERE, "synth_host.c")
_DEV_SRC = os.path.join(_HERE, "synth_dev.hip")
_HOST_LIB = os.path.join(_HERE, "libengram_synth_host.so")
_DEV_LIB = os.path.join(_HERE, "libengram_synth_dev.so")

ID_X, ID_KV, ID_W, ID_MASK, ID_GRAD, ID_EDGE, ID_ZERO = 1, 2, 3, 4, 5, 6, 7
# GateConv streams: H, k, v, dY, rms_w_h, rms_w_v, conv_w, edge-row choice
ID_GC_H, ID_GC_K, ID_GC_V, ID_GC_DY, ID_GC_WH, ID_GC_WV, ID_GC_CW, ID_GC_EDGE = 41, 42, 43, 44, 45, 46, 47, 48
D = 5120
S = 4

HIPCC_FLAGS = ["--offload-arch=gfx950", "-O3", "-fPIC", "-shared", "-std=c++17",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build_host(force: bool = False) -> str:
    if force or not os.path.exists(_HOST_LIB):
        tmp = _HOST_LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                               "-Wall", "-Wextra", "-o", tmp, _HOST_SRC, "-lm", "-lpthread"])
        os.replace(tmp, _HOST_LIB)
    return _HOST_LIB


def build_dev(force: bool = False) -> str:
    if force or not os.path.exists(_DEV_LIB):
        tmp = _DEV_LIB + ".tmp"
        subprocess.check_call(["hipcc", *HIPCC_FLAGS, "-o", tmp, _DEV_SRC],
                              stderr=subprocess.DEVNULL if not force else None)
        os.replace(tmp, _DEV_LIB)
    return _DEV_LIB


def build(force: bool = False) -> None:
    build_host(force)
    build_dev(force)


_host = None
_dev = None


def _h():
    global _host
    if _host is None:
        # ENGRAM_SYNTH_HOST_LIB names another build of synth_host.c (the
        # sanitizer test loads an instrumented one)
        lib = ctypes.CDLL(os.environ.get("ENGRAM_SYNTH_HOST_LIB") or build_host())
        P, I64, U64, U32, I = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32,
                               ctypes.c_int)
        lib.synth_stream_key.argtypes = [U64, U32]
        lib.synth_stream_key.restype = U64
        lib.synth_word.argtypes = [U64, U64]
        lib.synth_word.restype = U64
        lib.synth_normal_bf16.argtypes = [P, I64, U64, U32, I64, I]
        lib.synth_normal_f32.argtypes = [P, I64, U64, U32, I64, ctypes.c_float, ctypes.c_float, I]
        lib.synth_mask.argtypes = [P, I64, U64, U32, I64, U32, I]
        lib.synth_edge_rows.argtypes = [P, P, I64, I64, I64, I64, U64, U32, U32, P]
        lib.synth_zero_rows.argtypes = [I64, U64, P]
        for f in (lib.synth_normal_bf16, lib.synth_normal_f32, lib.synth_mask, lib.synth_edge_rows,
                  lib.synth_zero_rows):
            f.restype = None
        _host = lib
    return _host


def _d():
    global _dev
    if _dev is None:
        if not os.path.exists(_DEV_LIB):
            raise RuntimeError(f"device generator not built: {_DEV_LIB} (run __graft_entry__.build())")
        import torch  # noqa: F401  (bind to the HIP runtime torch loaded)
        lib = ctypes.CDLL(_DEV_LIB)
        P, I64, U64, U32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32
        lib.synth_dev_normal_bf16.argtypes = [P, I64, U64, U32, I64, P]
        lib.synth_dev_mask.argtypes = [P, I64, U64, U32, I64, U32, P]
        lib.synth_dev_normal_bf16.restype = ctypes.c_int
        lib.synth_dev_mask.restype = ctypes.c_int
        _dev = lib
    return _dev


def threshold(p: float) -> int:
    """24-bit Bernoulli threshold for probability p."""
    return int(round(p * (1 << 24)))


def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return 1


# ---------------- host generation (numpy) ----------------

def stream_key(seed: int, tid: int) -> int:
    return int(_h().synth_stream_key(seed, tid))


def word(key: int, c: int) -> int:
    return int(_h().synth_word(key, c))


def normal_bf16(count: int, seed: int, tid: int, offset: int = 0) -> np.ndarray:
    out = np.empty(count, np.uint16)
    if count:
        _h().synth_normal_bf16(out.ctypes.data, count, seed, tid, offset, _threads())
    return out


def normal_f32(count: int, seed: int, tid: int, mu: float, sigma: float, offset: int = 0) -> np.ndarray:
    out = np.empty(count, np.float32)
    if count:
        _h().synth_normal_f32(out.ctypes.data, count, seed, tid, offset, mu, sigma, _threads())
    return out


def mask(count: int, seed: int, p: float, offset: int = 0, tid: int = ID_MASK) -> np.ndarray:
    out = np.empty(count, np.uint8)
    if count:
        _h().synth_mask(out.ctypes.data, count, seed, tid, offset, threshold(p), _threads())
    return out


def apply_edge_rows(x16: np.ndarray, kv16: np.ndarray, n_total: int, t0: int, seed: int,
                    p_eps: float = 0.05, p_clamp: float = 0.10) -> np.ndarray:
    """In-place edge-row recipe on tokens [t0, t0 + len(x16)); returns per-kind counts."""
    assert x16.flags["C_CONTIGUOUS"] and kv16.flags["C_CONTIGUOUS"]
    nt = x16.shape[0]
    d = x16.shape[-1]
    counts = np.zeros(4, np.int64)
    _h().synth_edge_rows(x16.ctypes.data, kv16.ctypes.data, d, n_total, t0, nt, seed,
                         threshold(p_eps), threshold(p_clamp), counts.ctypes.data)
    return counts


def zero_rows(n_total: int, seed: int) -> np.ndarray:
    rows = np.empty(16, np.int64)
    _h().synth_zero_rows(n_total, seed, rows.ctypes.data)
    return rows


def host_inputs(n: int, seed: int = 0, p: float = 0.9, t0: int = 0, nt: int | None = None,
                d: int = D, grad: bool = False, edge: bool = False, n_total: int | None = None):
    """Tokens [t0, t0+nt) of the n-token workload, as numpy storage arrays.

    X [nt,4,d] bf16 bits, KV [nt,5d] bf16 bits, weight [4,d] fp32 N(1,0.1),
    mask [nt] Bernoulli(p), optionally grad_out [nt,4,d] bf16 bits and the
    edge-row recipe (which depends on the whole batch size n).
    """
    nt = n - t0 if nt is None else nt
    n_total = n if n_total is None else n_total
    x = normal_bf16(nt * S * d, seed, ID_X, t0 * S * d).reshape(nt, S, d)
    kv = normal_bf16(nt * 5 * d, seed, ID_KV, t0 * 5 * d).reshape(nt, 5 * d)
    w = normal_f32(S * d, seed, ID_W, 1.0, 0.1).reshape(S, d)
    m = mask(nt, seed, p, t0)
    res = {"x": x, "kv": kv, "weight": w, "mask": m}
    if edge:
        res["edge_counts"] = apply_edge_rows(x, kv, n_total, t0, seed)
    if grad:
        res["grad_out"] = normal_bf16(nt * S * d, seed, ID_GRAD, t0 * S * d).reshape(nt, S, d)
    return res


# ---------------- device generation (torch tensors as plain device memory) ----------------

def dev_normal_bf16(t, seed: int, tid: int, offset: int = 0) -> None:
    """Fill a contiguous 16-byte-aligned device tensor (2-byte elements) in place."""
    import torch
    assert t.is_cuda and t.is_contiguous() and t.element_size() == 2
    rc = _d().synth_dev_normal_bf16(t.data_ptr(), t.numel(), seed, tid, offset,
                                    torch.cuda.current_stream(t.device).cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_dev_normal_bf16 failed: hip error {rc}")


def dev_mask(t, seed: int, p: float, offset: int = 0, tid: int = ID_MASK) -> None:
    import torch
    assert t.is_cuda and t.is_contiguous() and t.element_size() == 1
    rc = _d().synth_dev_mask(t.data_ptr(), t.numel(), seed, tid, offset, threshold(p),
                             torch.cuda.current_stream(t.device).cuda_stream)
    if rc != 0:
        raise RuntimeError(f"synth_dev_mask failed: hip error {rc}")


def gateconv_inputs(M: int, T: int, d: int, seed: int = 0, edge: bool = False) -> dict:
    """GateConv inputs: H, k, v, dY [M,T,d] bf16 bits of N(0,1); rms_w_h,
    rms_w_v [d] fp32 of N(1, 0.25^2); conv_w [4,d] fp32 of N(0, 0.5^2).

    edge=True adds the degenerate rows of the map: a row r with word % 17 == 0
    gets H = k = 0 (alpha = 1/2 from eps alone), == 1 gets k = H (alpha
    saturates at 1 in fp32), == 2 gets v = 0 (vhat = 0, rrms_v = eps^-1/2)."""
    n = M * T * d
    res = {
        "H": normal_bf16(n, seed, ID_GC_H).reshape(M, T, d),
        "k": normal_bf16(n, seed, ID_GC_K).reshape(M, T, d),
        "v": normal_bf16(n, seed, ID_GC_V).reshape(M, T, d),
        "dY": normal_bf16(n, seed, ID_GC_DY).reshape(M, T, d),
        "wh": normal_f32(d, seed, ID_GC_WH, 1.0, 0.25),
        "wv": normal_f32(d, seed, ID_GC_WV, 1.0, 0.25),
        "cw": normal_f32(4 * d, seed, ID_GC_CW, 0.0, 0.5).reshape(4, d),
    }
    if edge:
        key = stream_key(seed, ID_GC_EDGE)
        H, k, v = (res[x].reshape(M * T, d) for x in ("H", "k", "v"))
        for r in range(M * T):
            kind = word(key, r) % 17
            if kind == 0:
                H[r] = 0
                k[r] = 0
            elif kind == 1:
                k[r] = H[r]
            elif kind == 2:
                v[r] = 0
    return res
