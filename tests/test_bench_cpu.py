"""Host-side logic of bench.py: algorithmic byte counts, the recorded-traffic
lookup and its invalidation, and the one-GPU guard.  No GPU needed."""
from __future__ import annotations

import importlib.util
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench(root=ROOT):
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(root, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_gate_byte_counts():
    b = load_bench()
    d, s = 5120, 4
    x = s * d * 2            # X row, bf16
    kv = (s + 1) * d * 2     # four keys and the shared value, bf16
    fwd = x + kv + 1 + x + s * 4 * 4          # + mask byte; out; saved (4 fp32 per stream)
    bwd = x + kv + x + s * 4 * 4 + x + kv     # X, KV, grad_out, saved; grad_x, grad_kv
    assert b.FWD_BYTES_PER_TOKEN == fwd == 133_185
    assert b.BWD_BYTES_PER_TOKEN == bwd == 225_344
    assert b.fwd_bytes(8192) == fwd * 8192 + s * d * 4
    assert b.bwd_bytes(8192) == bwd * 8192 + 2 * s * d * 4


def test_gateconv_byte_counts():
    b = load_bench()
    M, T, d = 4, 4096, 5120
    row_fwd = 3 * 2 * d + 2 * 2 * d + 4 * 4     # H, k, v in; Y, vhat out; four fp32 scalars out
    row_bwd = 5 * 2 * d + 4 * 4 + 3 * 2 * d     # dY, H, k, v, vhat and the scalars in; dH, dk, dv out
    weights = (1 + 1 + 4) * d * 4                # rms_w_h, rms_w_v, conv_w
    assert b.gc_fwd_bytes(M, T, d) == M * T * row_fwd + weights
    assert b.gc_bwd_bytes(M, T, d) == M * T * row_bwd + 2 * weights


def test_recorded_traffic_lookup():
    """A record is returned exactly when it was taken on the current sources;
    a stale one (kernel edited since the counters were taken) reads as None,
    which the benchmark reports as null traffic."""
    b = load_bench()
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    stale = []
    for k in b.KERNEL_SOURCES:
        assert k in rec, k
        fresh = rec[k]["source_hash"] == b.kernel_source_hash(k)
        assert b.recorded_traffic(k) == (rec[k]["bytes_per_launch"] if fresh else None), k
        if not fresh:
            stale.append(k)
    if stale:
        pytest.skip(f"traffic counters predate the current sources of {stale}")


def test_recorded_traffic_invalidated_by_a_source_change(tmp_path):
    root = tmp_path / "repo"
    (root / "memory_bound_engram_amd" / "csrc").mkdir(parents=True)
    (root / "profiles").mkdir()
    shutil.copy(os.path.join(ROOT, "bench.py"), root / "bench.py")
    for name in ("engram_device.h", "engram_fwd.hip", "engram_bwd.hip", "engram_gateconv.hip", "engram_api.cpp"):
        shutil.copy(os.path.join(ROOT, "memory_bound_engram_amd", "csrc", name),
                    root / "memory_bound_engram_amd" / "csrc" / name)
    b = load_bench(str(root))
    # a record taken on exactly these sources, whatever the committed one's age
    rec = {k: {"source_hash": b.kernel_source_hash(k), "bytes_per_launch": 1000 + i}
           for i, k in enumerate(b.KERNEL_SOURCES)}
    with open(root / "profiles" / "traffic.json", "w") as f:
        json.dump(rec, f)
    assert b.recorded_traffic("bwd") == rec["bwd"]["bytes_per_launch"]
    bwd_src = root / "memory_bound_engram_amd" / "csrc" / "engram_bwd.hip"
    with open(bwd_src, "a") as f:  # comments and layout are not code: the record stands
        f.write("\n// a comment\n/* another\n   one */   \n")
    assert b.recorded_traffic("bwd") == rec["bwd"]["bytes_per_launch"]
    with open(bwd_src, "a") as f:  # a code edit voids it
        f.write("static const int engram_edited = 1;\n")
    assert b.recorded_traffic("bwd") is None
    assert b.recorded_traffic("fwd") == rec["fwd"]["bytes_per_launch"]  # other kernels keep their record


def test_code_only_strips_comments_not_literals():
    b = load_bench()
    src = 'int a = 1;  // one\n/* two\n */ const char* s = "x // y /* z */";\nchar q = \'\\\'\';\n'
    assert b.code_only(src) == 'int a = 1; const char* s = "x // y /* z */"; char q = \'\\\'\';'
    assert b.code_only("a/b") == "a/b" and b.code_only("a /*x*/b") == "a b"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""
