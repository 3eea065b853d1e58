"""The host C code under AddressSanitizer and UndefinedBehaviorSanitizer.

The fp64 oracle (oracle/engram_oracle.c) and the host input generator
(synth/synth_host.c) are rebuilt with gcc and -fsanitize=address,undefined
in a temporary directory, and the oracle, tolerance-scale, GateConv,
random-case property and generator pin suites run against those builds in a child process with the
sanitizer runtimes preloaded (the Python interpreter itself is not
instrumented).  Any out-of-bounds access, use after free or undefined
operation in the C code aborts the child; the test also refuses a run whose
output mentions a sanitizer report.  Host code only: nothing here touches a
GPU.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def test_oracle_and_generator_clean_under_asan_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    builds = {}
    for name, src in (("oracle", os.path.join(ROOT, "oracle", "engram_oracle.c")),
                      ("synth", os.path.join(ROOT, "synth", "synth_host.c"))):
        lib = tmp_path / f"lib{name}_san.so"
        subprocess.check_call(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared", *SAN,
                               "-o", str(lib), src, "-lm", "-lpthread"])
        builds[name] = str(lib)
    env = dict(os.environ,
               ENGRAM_ORACLE_LIB=builds["oracle"], ENGRAM_SYNTH_HOST_LIB=builds["synth"],
               LD_PRELOAD=f"{asan}:{ubsan}",
               # CPython keeps objects alive at exit by design: leak reports would be noise
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_tolerance_scales.py"),
                        os.path.join(ROOT, "tests", "test_oracle_gateconv_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_property_cpu.py"),
                        os.path.join(ROOT, "tests", "test_oracle_gateconv_property_cpu.py"),
                        os.path.join(ROOT, "tests", "test_synth.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout + r.stderr
    assert r.returncode == 0, f"pins failed under the sanitizers:\n{out[-4000:]}"
    for marker in ("ERROR: AddressSanitizer", "runtime error:", "SUMMARY: UndefinedBehaviorSanitizer"):
        assert marker not in out, f"sanitizer report:\n{out[-4000:]}"
    assert " passed" in out


def test_harness_reports_a_planted_overflow(tmp_path):
    """Control: the same build flags and preload catch a heap overflow in a
    ctypes-loaded library, so a clean run above means something."""
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not (asan and ubsan):
        pytest.skip("gcc sanitizer runtimes not installed")
    src = tmp_path / "overflow.c"
    src.write_text("#include <stdlib.h>\n"
                   "int overflow(int n) { int *p = malloc(n * sizeof(int)); p[n] = 1; int r = p[0]; free(p); return r; }\n")
    lib = tmp_path / "liboverflow.so"
    subprocess.check_call(["gcc", "-O1", "-g", "-fPIC", "-shared", *SAN, "-o", str(lib), str(src)])
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    code = f"import ctypes; ctypes.CDLL({str(lib)!r}).overflow(4)"
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "AddressSanitizer: heap-buffer-overflow" in r.stderr
