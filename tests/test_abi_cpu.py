"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/engram.h declares, sizes the workspace by the page's formula, and
rejects every invalid call on the host before any HIP call (fake device
addresses are used, so an accepted call would be a bug)."""
from __future__ import annotations

import ctypes
import json
import os
import re

import pytest

import memory_bound_engram_amd as eg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "engram.h")
GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "gate_spec_constants.json")))

XB = 4 * 5120 * 2       # bytes per token of x / out / grad
KVB = 25600 * 2         # bytes per token of kv
WB = 4 * 5120 * 4       # weight bytes
SB = 64                 # saved bytes per token


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(engram_\w+)\s*\(", text)))


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("engram_gate_fwd", "engram_gate_bwd", "engram_gate_bwd_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(eg.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), f"{name} declared in engram.h but not exported"


def test_header_constants_match_the_page():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define (ENGRAM_\w+) (\d+)", text))
    assert int(consts["ENGRAM_STREAMS"]) == GOLDEN["streams"]["value"]
    assert int(consts["ENGRAM_HIDDEN"]) == GOLDEN["hidden"]["value"]
    assert int(consts["ENGRAM_KV_COLS"]) == GOLDEN["kv_columns"]["value"]
    assert int(consts["ENGRAM_N_MAX"]) == GOLDEN["n_max"]["value"]
    assert int(consts["ENGRAM_BWD_N_MAX"]) == GOLDEN["bwd_n_max"]["value"]
    assert int(consts["ENGRAM_BWD_N_MULTIPLE"]) == GOLDEN["bwd_n_multiple"]["value"]


@pytest.mark.parametrize("n", [0, -5, 1, 63, 64, 100, 4096, 8192, 8256, 1 << 20])
def test_workspace_formula(n):
    want = 4 * (16 * n + 4 * 5120 * (n // 64)) if n > 0 else 0
    assert eg.engram_gate_bwd_workspace_bytes(n) == want


def test_workspace_worked_values():
    assert eg.engram_gate_bwd_workspace_bytes(64) == 86016
    assert eg.engram_gate_bwd_workspace_bytes(4096) == 5505024
    assert eg.engram_gate_bwd_workspace_bytes(8192) == 11010048


# ---------------- forward validation ----------------

BASE = 1 << 40  # fake, 16-byte-aligned, never dereferenced


def fwd_layout(n):
    x = BASE
    kv = x + n * XB + 4096
    w = kv + n * KVB + 4096
    m = w + WB + 4096
    out = m + n + 4096 + 16
    out -= out % 16
    sv = out + n * XB + 4096
    return dict(x=x, kv=kv, w=w, m=m, out=out, sv=sv)


def call_fwd(a, n):
    return eg.lib.engram_gate_fwd(a["x"], a["kv"], a["w"], a["m"], a["out"], a["sv"], n, None)


@pytest.mark.parametrize("field", ["x", "kv", "w", "m", "out"])
def test_fwd_rejects_null(field):
    a = fwd_layout(8)
    a[field] = None
    assert call_fwd(a, 8) == eg.ERR_NULL


def test_fwd_without_saved_is_still_validated():
    # saved == NULL selects the inference forward; everything else is checked
    a = fwd_layout(8)
    a["sv"] = None
    a["x"] += 4
    assert call_fwd(a, 8) == eg.ERR_ALIGN
    a = fwd_layout(8)
    a["sv"] = None
    a["out"] = a["kv"]
    assert call_fwd(a, 8) == eg.ERR_OVERLAP
    assert call_fwd(dict(fwd_layout(8), sv=None), 0) == eg.ERR_N_RANGE


@pytest.mark.parametrize("n", [0, -1, 4194241, 1 << 40])
def test_fwd_rejects_n_out_of_range(n):
    assert call_fwd(fwd_layout(8), n) == eg.ERR_N_RANGE


@pytest.mark.parametrize("field", ["x", "kv", "w", "out", "sv"])
def test_fwd_rejects_misaligned(field):
    a = fwd_layout(8)
    a[field] += 2
    assert call_fwd(a, 8) == eg.ERR_ALIGN


def test_fwd_mask_may_be_unaligned_but_overlap_is_checked():
    a = fwd_layout(8)
    a["out"] = a["x"]  # out aliases x
    assert call_fwd(a, 8) == eg.ERR_OVERLAP
    a = fwd_layout(8)
    a["sv"] = a["out"] + 8 * XB - 16  # saved overlaps the tail of out
    assert call_fwd(a, 8) == eg.ERR_OVERLAP
    a = fwd_layout(8)
    a["out"] = a["m"] - (a["m"] % 16)  # out starts inside the mask bytes
    assert call_fwd(a, 8) == eg.ERR_OVERLAP
    a = fwd_layout(8)
    a["sv"] = a["w"] + WB - 16  # saved overlaps the weight
    assert call_fwd(a, 8) == eg.ERR_OVERLAP


# ---------------- backward validation ----------------

def bwd_layout(n):
    p = BASE
    a = {}
    for name, size in (("x", n * XB), ("kv", n * KVB), ("w", WB), ("sv", n * SB), ("g", n * XB),
                       ("dx", n * XB), ("dkv", n * KVB), ("dw", WB),
                       ("ws", max(eg.engram_gate_bwd_workspace_bytes(n), 16))):
        a[name] = p
        p += size + 4096
    return a


def call_bwd(a, n):
    return eg.lib.engram_gate_bwd(a["x"], a["kv"], a["w"], a["sv"], a["g"], a["dx"], a["dkv"], a["dw"],
                                  a["ws"], n, None)


@pytest.mark.parametrize("field", ["x", "kv", "w", "sv", "g", "dx", "dkv", "dw", "ws"])
def test_bwd_rejects_null(field):
    a = bwd_layout(64)
    a[field] = None
    assert call_bwd(a, 64) == eg.ERR_NULL


@pytest.mark.parametrize("n,code", [(0, eg.ERR_N_RANGE), (-64, eg.ERR_N_RANGE), (8256, eg.ERR_N_RANGE),
                                    (100, eg.ERR_N_MULT64), (1, eg.ERR_N_MULT64), (8191, eg.ERR_N_MULT64)])
def test_bwd_rejects_bad_n(n, code):
    assert call_bwd(bwd_layout(max(n, 64)), n) == code


@pytest.mark.parametrize("field", ["x", "kv", "w", "sv", "g", "dx", "dkv", "dw", "ws"])
def test_bwd_rejects_misaligned(field):
    a = bwd_layout(64)
    a[field] += 8
    assert call_bwd(a, 64) == eg.ERR_ALIGN


@pytest.mark.parametrize("out,other", [("dx", "x"), ("dx", "g"), ("dkv", "kv"), ("dw", "w"), ("ws", "sv"),
                                       ("dx", "dkv"), ("ws", "dw"), ("dkv", "ws")])
def test_bwd_rejects_overlap(out, other):
    a = bwd_layout(64)
    a[out] = a[other]
    assert call_bwd(a, 64) == eg.ERR_OVERLAP


def test_bwd_inputs_may_alias_each_other():
    # grad_out aliasing x is legal; with fake addresses the call then fails only
    # at launch, so check validation alone via an overlap that is still caught.
    a = bwd_layout(64)
    a["g"] = a["x"]
    a["dx"] = a["x"]
    assert call_bwd(a, 64) == eg.ERR_OVERLAP


def test_status_strings():
    for s in range(7):
        assert eg.lib.engram_status_string(s)


# ---------------- the allocation-free backward (no workspace argument) ----------------

def call_na(a, n):
    return eg.lib.engram_gate_bwd_noalloc(a["x"], a["kv"], a["w"], a["sv"], a["g"], a["dx"], a["dkv"], a["dw"],
                                          n, None)


@pytest.mark.parametrize("field", ["x", "kv", "w", "sv", "g", "dx", "dkv", "dw"])
def test_noalloc_rejects_null(field):
    a = bwd_layout(64)
    a[field] = None
    assert call_na(a, 64) == eg.ERR_NULL


@pytest.mark.parametrize("n,code", [(0, eg.ERR_N_RANGE), (-64, eg.ERR_N_RANGE), (8256, eg.ERR_N_RANGE),
                                    (1 << 20, eg.ERR_N_RANGE), (100, eg.ERR_N_MULT64), (8191, eg.ERR_N_MULT64)])
def test_noalloc_rejects_sizes_beyond_its_array(n, code):
    assert call_na(bwd_layout(max(n, 64)), n) == code


def test_noalloc_limit_matches_header():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define (ENGRAM_NOALLOC_\w+) (\d+)", text))
    assert int(consts["ENGRAM_NOALLOC_N_MAX"]) == eg.NOALLOC_N_MAX == 8192
    assert int(consts["ENGRAM_NOALLOC_SCRATCH_BYTES"]) == (8192 // 64) * 4 * 5120 * 4


@pytest.mark.parametrize("field", ["x", "kv", "w", "sv", "g", "dx", "dkv", "dw"])
def test_noalloc_rejects_misaligned(field):
    a = bwd_layout(64)
    a[field] += 8
    assert call_na(a, 64) == eg.ERR_ALIGN


@pytest.mark.parametrize("out,other", [("dx", "x"), ("dx", "g"), ("dkv", "kv"), ("dw", "w"), ("dw", "sv"),
                                       ("dx", "dkv"), ("dkv", "dw")])
def test_noalloc_rejects_overlap(out, other):
    a = bwd_layout(64)
    a[out] = a[other]
    assert call_na(a, 64) == eg.ERR_OVERLAP


# ---------------- backward with the product rule; fused weight ----------------

def nw_layout(n):
    a = bwd_layout(n)
    p = max(a.values()) + (1 << 30)
    for name, size in (("wh", WB // 2), ("we", WB // 2), ("gwh", WB), ("gwe", WB)):
        a[name] = p
        p += size + 4096
    return a


def call_nw(a, n):
    return eg.lib.engram_gate_bwd_with_norm_weights(a["x"], a["kv"], a["w"], a["sv"], a["g"], a["dx"], a["dkv"],
                                                    a["dw"], a["wh"], a["we"], a["gwh"], a["gwe"], a["ws"], n,
                                                    None)


@pytest.mark.parametrize("field", ["wh", "we", "gwh", "gwe", "x", "ws"])
def test_bwd_norm_weights_rejects_null(field):
    a = nw_layout(64)
    a[field] = None
    assert call_nw(a, 64) == eg.ERR_NULL


@pytest.mark.parametrize("field", ["wh", "we", "gwh", "gwe"])
def test_bwd_norm_weights_rejects_misaligned(field):
    a = nw_layout(64)
    a[field] += 2
    assert call_nw(a, 64) == eg.ERR_ALIGN


@pytest.mark.parametrize("out,other", [("gwh", "wh"), ("gwe", "we"), ("gwh", "gwe"), ("gwh", "dw"),
                                       ("gwe", "x"), ("dx", "wh")])
def test_bwd_norm_weights_rejects_overlap(out, other):
    a = nw_layout(64)
    a[out] = a[other]
    assert call_nw(a, 64) == eg.ERR_OVERLAP


def test_bwd_norm_weights_checks_n():
    assert call_nw(nw_layout(64), 100) == eg.ERR_N_MULT64
    assert call_nw(nw_layout(64), 8256) == eg.ERR_N_RANGE


def test_fused_weight_validation():
    f = eg.lib.engram_fused_weight
    wh, we, w = BASE, BASE + (1 << 20), BASE + (2 << 20)
    assert f(None, we, w, None) == eg.ERR_NULL
    assert f(wh, None, w, None) == eg.ERR_NULL
    assert f(wh, we, None, None) == eg.ERR_NULL
    assert f(wh + 2, we, w, None) == eg.ERR_ALIGN
    assert f(wh, we, w + 8, None) == eg.ERR_ALIGN
    assert f(wh, we, wh, None) == eg.ERR_OVERLAP
    assert f(wh, we, we + 1024, None) == eg.ERR_OVERLAP


# ---------------- GateConv ----------------

def gc_chunk(rows, d):
    """Rows per workgroup chunk of the backward (which sizes its workspace)."""
    nw = d // 512
    waves = 4 if nw in (3, 5) else nw  # d = 1536 and 2560 run the backward on 768 x 2 and 256 x 10 maps
    target = 256 * (1 if waves >= 8 else 8 // waves)
    return min(max(-(-rows // target), 16 if nw <= 2 else 32), 512)


@pytest.mark.parametrize("M,T,d", [(1, 1, 512), (2, 45, 512), (3, 300, 1024), (2, 37, 5120), (4, 2048, 5120),
                                   (8, 4096, 5120), (1, 4194304, 512), (4, 4096, 1536), (4, 4096, 2560),
                                   (1, 100000, 1536), (3, 33, 2560),
                                   (0, 4, 512), (1, 0, 512), (1, 1, 0), (1, 1, 640), (1, 1, 5632), (2, 2097153, 512)])
def test_gateconv_workspace_formula(M, T, d):
    rows = M * T
    ok = M >= 1 and T >= 1 and rows <= 4194304 and d >= 512 and d % 512 == 0 and d <= 5120
    nwg = -(-rows // gc_chunk(rows, d)) if ok else 0
    want = ((nwg + -(-nwg // 64)) * 5 * d * 4 + 4 * rows) if ok else 0  # partials, their 64-row sums, ds
    assert eg.engram_gateconv_bwd_workspace_bytes(M, T, d) == want


def gc_fwd_layout(M, T, d):
    tb, sb = M * T * d * 2, M * T * 4
    a, p = {}, BASE
    for name, size in (("H", tb), ("k", tb), ("v", tb), ("wh", 4 * d), ("wv", 4 * d), ("cw", 16 * d), ("Y", tb),
                       ("vhat", tb), ("alpha", sb), ("rh", sb), ("rk", sb), ("rv", sb)):
        a[name] = p
        p += size + 4096
    return a


def call_gc_fwd(a, M, T, d, eps=1e-6):
    return eg.lib.engram_gateconv_fwd(a["H"], a["k"], a["v"], a["wh"], a["wv"], a["cw"], a["Y"], a["vhat"],
                                      a["alpha"], a["rh"], a["rk"], a["rv"], M, T, d, eps, None)


GC_FWD_FIELDS = ["H", "k", "v", "wh", "wv", "cw", "Y", "vhat", "alpha", "rh", "rk", "rv"]


@pytest.mark.parametrize("field", GC_FWD_FIELDS)
def test_gateconv_fwd_rejects_null(field):
    a = gc_fwd_layout(2, 8, 512)
    a[field] = None
    assert call_gc_fwd(a, 2, 8, 512) == eg.ERR_NULL


@pytest.mark.parametrize("field", GC_FWD_FIELDS)
def test_gateconv_fwd_rejects_misaligned(field):
    a = gc_fwd_layout(2, 8, 512)
    a[field] += 4
    assert call_gc_fwd(a, 2, 8, 512) == eg.ERR_ALIGN


@pytest.mark.parametrize("M,T,d,eps", [(0, 8, 512, 1e-6), (2, 0, 512, 1e-6), (-1, 8, 512, 1e-6), (2, 8, 256, 1e-6),
                                       (2, 8, 1000, 1e-6), (2, 8, 5632, 1e-6), (4097, 1024, 512, 1e-6),
                                       (2, 8, 512, -1e-6), (2, 8, 512, float("nan")), (2, 8, 512, 2.0)])
def test_gateconv_fwd_rejects_bad_sizes(M, T, d, eps):
    assert call_gc_fwd(gc_fwd_layout(2, 8, 512), M, T, d, eps) == eg.ERR_N_RANGE


@pytest.mark.parametrize("out,other", [("Y", "H"), ("vhat", "v"), ("alpha", "wh"), ("rv", "cw"), ("Y", "vhat"),
                                       ("rh", "rk"), ("alpha", "Y")])
def test_gateconv_fwd_rejects_overlap(out, other):
    a = gc_fwd_layout(2, 8, 512)
    a[out] = a[other]
    assert call_gc_fwd(a, 2, 8, 512) == eg.ERR_OVERLAP


def gc_bwd_layout(M, T, d):
    tb, sb = M * T * d * 2, M * T * 4
    a, p = {}, BASE
    for name, size in (("dY", tb), ("H", tb), ("k", tb), ("v", tb), ("wh", 4 * d), ("wv", 4 * d), ("cw", 16 * d),
                       ("vhat", tb), ("alpha", sb), ("rh", sb), ("rk", sb), ("rv", sb), ("dH", tb), ("dk", tb),
                       ("dv", tb), ("dwh", 4 * d), ("dwv", 4 * d), ("dcw", 16 * d),
                       ("ws", eg.engram_gateconv_bwd_workspace_bytes(M, T, d))):
        a[name] = p
        p += size + 4096
    return a


GC_BWD_FIELDS = ["dY", "H", "k", "v", "wh", "wv", "cw", "vhat", "alpha", "rh", "rk", "rv", "dH", "dk", "dv", "dwh",
                 "dwv", "dcw", "ws"]


def call_gc_bwd(a, M, T, d):
    return eg.lib.engram_gateconv_bwd(*[a[f] for f in GC_BWD_FIELDS], M, T, d, None)


@pytest.mark.parametrize("field", GC_BWD_FIELDS)
def test_gateconv_bwd_rejects_null(field):
    a = gc_bwd_layout(2, 40, 1024)
    a[field] = None
    assert call_gc_bwd(a, 2, 40, 1024) == eg.ERR_NULL


@pytest.mark.parametrize("field", GC_BWD_FIELDS)
def test_gateconv_bwd_rejects_misaligned(field):
    a = gc_bwd_layout(2, 40, 1024)
    a[field] += 8
    assert call_gc_bwd(a, 2, 40, 1024) == eg.ERR_ALIGN


@pytest.mark.parametrize("M,T,d", [(0, 40, 1024), (2, 0, 1024), (2, 40, 1000), (2, 40, 6144), (5000, 1000, 512)])
def test_gateconv_bwd_rejects_bad_sizes(M, T, d):
    assert call_gc_bwd(gc_bwd_layout(2, 40, 1024), M, T, d) == eg.ERR_N_RANGE


@pytest.mark.parametrize("out,other", [("dH", "H"), ("dk", "dY"), ("dv", "vhat"), ("dwh", "wh"), ("dcw", "cw"),
                                       ("ws", "alpha"), ("dH", "dk"), ("dwv", "ws"), ("ws", "dv")])
def test_gateconv_bwd_rejects_overlap(out, other):
    a = gc_bwd_layout(2, 40, 1024)
    a[out] = a[other]
    assert call_gc_bwd(a, 2, 40, 1024) == eg.ERR_OVERLAP


def test_gateconv_bwd_workspace_tail_overlap():
    a = gc_bwd_layout(2, 40, 1024)
    a["dcw"] = a["ws"] + eg.engram_gateconv_bwd_workspace_bytes(2, 40, 1024) - 16
    assert call_gc_bwd(a, 2, 40, 1024) == eg.ERR_OVERLAP
