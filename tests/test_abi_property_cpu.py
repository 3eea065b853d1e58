"""Host-side validation of the gate's calls against a plain model of the
header's rules, over random arguments (hypothesis).

The model follows include/engram.h: NULL pointers first, then the size
limits ("Engram saved-state gate", layout paragraph: N <= 4,194,240; the
backward N <= 8192 and a multiple of 64), then 16-byte alignment of every
floating tensor and the workspace, then byte-range overlap of any output or
the workspace with any input or another output (saved-state paragraph);
inputs may alias each other, and an empty range (saved == NULL) overlaps
nothing.  Buffers are placed at fake addresses drawn from 24 slots, so
collisions and partial overlaps are common; at most one deliberate fault (a
NULL or a misaligned pointer) per draw.  Every rejected configuration must
come back with exactly the model's status.  A configuration the model accepts
is passed to the library only where no GPU is visible: validation passes and
the launch then fails (ENGRAM_ERR_LAUNCH), which shows nothing legal is
rejected; with a GPU it would launch kernels on fake pointers, so it is
skipped there.
"""
from __future__ import annotations

import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

import memory_bound_engram_amd as eg  # noqa: E402

XB, KVB, WB, SB = 4 * 5120 * 2, 25600 * 2, 4 * 5120 * 4, 64
BASE = 1 << 40
SPAN = 1 << 32  # room for the largest range the tests draw
ACCEPT = "accept"


def _overlaps(a, b):
    return a[0] < a[1] and b[0] < b[1] and a[0] < b[1] and b[0] < a[1]


def _any_overlap(ins, outs):
    for i, o in enumerate(outs):
        if any(_overlaps(o, r) for r in ins) or any(_overlaps(o, r) for r in outs[i + 1:]):
            return True
    return False


def _rng(p, size):
    return (p, p + size) if p is not None else (0, 0)


def _no_gpu():
    import torch
    return torch.cuda.device_count() == 0  # counts devices without starting the runtime


@st.composite
def _layout(draw, names, nullable, slots=24):
    """Fake 16-byte-aligned addresses in `slots` slots (so some buffers share a
    slot and overlap), then at most one fault: a NULL (among `nullable`) or a
    misaligned pointer."""
    a = {}
    for k in names:
        a[k] = BASE + draw(st.integers(0, slots - 1)) * SPAN + 16 * draw(st.integers(0, 1 << 16))
    fault = draw(st.sampled_from(["none"] * 4 + ["null", "align"]))
    k = draw(st.sampled_from(names))
    if fault == "null" and k in nullable:
        a[k] = None
    elif fault == "align":
        a[k] += draw(st.sampled_from([1, 2, 4, 8]))
    return a


_N_FWD = st.one_of(st.integers(-3, 0), st.integers(1, 300), st.sampled_from([4194240, 4194241, 1 << 33]))
_N_BWD = st.one_of(st.integers(-64, 0), st.sampled_from([1, 63, 64, 100, 128, 4096, 8128, 8191, 8192, 8256, 1 << 20]),
                   st.integers(1, 130).map(lambda k: 64 * k))


def _fwd_model(a, n):
    if any(a[k] is None for k in ("x", "kv", "w", "m", "out")):
        return eg.ERR_NULL
    if n < 1 or n > eg.N_MAX:
        return eg.ERR_N_RANGE
    if any(a[k] % 16 for k in ("x", "kv", "w", "out")) or (a["sv"] is not None and a["sv"] % 16):
        return eg.ERR_ALIGN
    ins = [_rng(a["x"], n * XB), _rng(a["kv"], n * KVB), _rng(a["w"], WB), _rng(a["m"], n)]
    outs = [_rng(a["out"], n * XB), _rng(a["sv"], n * SB)]
    return eg.ERR_OVERLAP if _any_overlap(ins, outs) else ACCEPT


def _bwd_model(a, n):
    if any(a[k] is None for k in a):
        return eg.ERR_NULL
    if n < 1 or n > eg.BWD_N_MAX:
        return eg.ERR_N_RANGE
    if n % eg.BWD_N_MULTIPLE:
        return eg.ERR_N_MULT64
    if any(a[k] % 16 for k in a):
        return eg.ERR_ALIGN
    ins = [_rng(a["x"], n * XB), _rng(a["kv"], n * KVB), _rng(a["w"], WB), _rng(a["sv"], n * SB),
           _rng(a["g"], n * XB)]
    outs = [_rng(a["dx"], n * XB), _rng(a["dkv"], n * KVB), _rng(a["dw"], WB),
            _rng(a["ws"], eg.engram_gate_bwd_workspace_bytes(n))]
    return eg.ERR_OVERLAP if _any_overlap(ins, outs) else ACCEPT


@settings(max_examples=600, deadline=None)
@given(st.data())
def test_fwd_validation_matches_the_model(data):
    names = ("x", "kv", "w", "m", "out", "sv")
    a = data.draw(_layout(names, names), label="layout")
    n = data.draw(_N_FWD, label="N")
    want = _fwd_model(a, n)
    if want == ACCEPT:
        if not _no_gpu():
            return  # a valid call would launch kernels on fake addresses
        want = eg.ERR_LAUNCH
    got = eg.lib.engram_gate_fwd(a["x"], a["kv"], a["w"], a["m"], a["out"], a["sv"], n, None)
    assert got == want, (a, n)


@settings(max_examples=600, deadline=None)
@given(st.data())
def test_bwd_validation_matches_the_model(data):
    names = ("x", "kv", "w", "sv", "g", "dx", "dkv", "dw", "ws")
    a = data.draw(_layout(names, names), label="layout")
    n = data.draw(_N_BWD, label="N")
    want = _bwd_model(a, n)
    if want == ACCEPT:
        if not _no_gpu():
            return
        want = eg.ERR_LAUNCH
    got = eg.lib.engram_gate_bwd(*(a[k] for k in names), n, None)
    assert got == want, (a, n)


@settings(max_examples=300, deadline=None)
@given(st.data())
def test_noalloc_validation_matches_the_model(data):
    """The allocation-free backward: the same rules without the workspace."""
    names = ("x", "kv", "w", "sv", "g", "dx", "dkv", "dw")
    a = data.draw(_layout(names, names), label="layout")
    n = data.draw(_N_BWD, label="N")
    # the model of the workspace call, with a workspace far from everything
    want = _bwd_model(dict(a, ws=BASE + 30 * SPAN), n)
    if want == ACCEPT:
        if not _no_gpu():
            return
        want = eg.ERR_LAUNCH
    got = eg.lib.engram_gate_bwd_noalloc(*(a[k] for k in names), n, None)
    assert got == want, (a, n)


def test_the_model_accepts_some_and_rejects_each_way():
    """The random draws reach every outcome (checked on fixed draws here)."""
    ok = {k: BASE + i * SPAN for i, k in enumerate(("x", "kv", "w", "m", "out", "sv"))}
    assert _fwd_model(ok, 8) == ACCEPT
    assert _fwd_model(dict(ok, sv=None), 8) == ACCEPT
    assert _fwd_model(dict(ok, m=None), 8) == eg.ERR_NULL
    assert _fwd_model(ok, 0) == eg.ERR_N_RANGE
    assert _fwd_model(dict(ok, m=ok["m"] + 1), 8) == ACCEPT  # the mask needs no alignment
    assert _fwd_model(dict(ok, out=ok["out"] + 8), 8) == eg.ERR_ALIGN
    assert _fwd_model(dict(ok, sv=ok["x"] + XB), 8) == eg.ERR_OVERLAP


# ---------------- GateConv ("Engram Operators", GateConv section) ----------------

_GC_FWD = ("H", "k", "v", "wh", "wv", "cw", "Y", "vhat", "alpha", "rh", "rk", "rv")
_GC_BWD = ("dY", "H", "k", "v", "wh", "wv", "cw", "vhat", "alpha", "rh", "rk", "rv",
           "dH", "dk", "dv", "dwh", "dwv", "dcw", "ws")
_GC_VALID = st.tuples(st.integers(1, 8), st.integers(1, 600), st.integers(1, 10).map(lambda q: 512 * q))
_GC_DIMS = st.one_of(
    _GC_VALID, _GC_VALID, _GC_VALID,
    st.tuples(st.integers(-1, 3), st.integers(-1, 3), st.sampled_from([0, 511, 512, 640, 5120, 5632])),
    st.sampled_from([(1024, 4097, 512), (4194305, 1, 512), (1, 4194305, 512), (2048, 2048, 512)]))


def _gc_dims_ok(M, T, d):
    return (1 <= M <= eg.GATECONV_ROWS_MAX and 1 <= T <= eg.GATECONV_ROWS_MAX and M * T <= eg.GATECONV_ROWS_MAX
            and 512 <= d <= eg.GATECONV_D_MAX and d % 512 == 0)


def _gc_fwd_model(a, M, T, d, eps):
    if any(a[k] is None for k in _GC_FWD):
        return eg.ERR_NULL
    if not _gc_dims_ok(M, T, d) or not (0.0 <= eps <= 1.0):
        return eg.ERR_N_RANGE
    if any(a[k] % 16 for k in _GC_FWD):
        return eg.ERR_ALIGN
    tb, sb = M * T * d * 2, M * T * 4
    ins = [_rng(a["H"], tb), _rng(a["k"], tb), _rng(a["v"], tb), _rng(a["wh"], 4 * d), _rng(a["wv"], 4 * d),
           _rng(a["cw"], 16 * d)]
    outs = [_rng(a["Y"], tb), _rng(a["vhat"], tb)] + [_rng(a[k], sb) for k in ("alpha", "rh", "rk", "rv")]
    return eg.ERR_OVERLAP if _any_overlap(ins, outs) else ACCEPT


def _gc_bwd_model(a, M, T, d):
    if any(a[k] is None for k in _GC_BWD):
        return eg.ERR_NULL
    if not _gc_dims_ok(M, T, d):
        return eg.ERR_N_RANGE
    if any(a[k] % 16 for k in _GC_BWD):
        return eg.ERR_ALIGN
    tb, sb = M * T * d * 2, M * T * 4
    ins = ([_rng(a[k], tb) for k in ("dY", "H", "k", "v")] + [_rng(a["wh"], 4 * d), _rng(a["wv"], 4 * d),
           _rng(a["cw"], 16 * d), _rng(a["vhat"], tb)] + [_rng(a[k], sb) for k in ("alpha", "rh", "rk", "rv")])
    outs = ([_rng(a[k], tb) for k in ("dH", "dk", "dv")] + [_rng(a["dwh"], 4 * d), _rng(a["dwv"], 4 * d),
            _rng(a["dcw"], 16 * d), _rng(a["ws"], eg.engram_gateconv_bwd_workspace_bytes(M, T, d))])
    return eg.ERR_OVERLAP if _any_overlap(ins, outs) else ACCEPT


@settings(max_examples=500, deadline=None)
@given(st.data())
def test_gateconv_fwd_validation_matches_the_model(data):
    a = data.draw(_layout(_GC_FWD, _GC_FWD, slots=48), label="layout")
    M, T, d = data.draw(_GC_DIMS, label="M, T, d")
    eps = data.draw(st.sampled_from([1e-6, 0.0, 1.0, 0.5, -1e-6, 1.5, float("nan"), float("inf")]), label="eps")
    want = _gc_fwd_model(a, M, T, d, eps)
    if want == ACCEPT:
        if not _no_gpu():
            return
        want = eg.ERR_LAUNCH
    got = eg.lib.engram_gateconv_fwd(*(a[k] for k in _GC_FWD), M, T, d, eps, None)
    assert got == want, (a, M, T, d, eps)


@settings(max_examples=500, deadline=None)
@given(st.data())
def test_gateconv_bwd_validation_matches_the_model(data):
    a = data.draw(_layout(_GC_BWD, _GC_BWD, slots=96), label="layout")
    M, T, d = data.draw(_GC_DIMS, label="M, T, d")
    want = _gc_bwd_model(a, M, T, d)
    if want == ACCEPT:
        if not _no_gpu():
            return
        want = eg.ERR_LAUNCH
    got = eg.lib.engram_gateconv_bwd(*(a[k] for k in _GC_BWD), M, T, d, None)
    assert got == want, (a, M, T, d)
