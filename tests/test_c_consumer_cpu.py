"""The boundary is a plain C ABI: tests/abi_consumer.c, which includes only
include/engram.h (no HIP or Python headers), builds with gcc as C11 and with
g++ as C++17 under -Wall -Wextra -Werror -pedantic, links against
libengram.so, and checks every declared function's host-side behaviour
(status codes, size helpers) without a GPU."""
from __future__ import annotations

import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIBDIR = os.path.join(ROOT, "memory_bound_engram_amd")
SRC = os.path.join(ROOT, "tests", "abi_consumer.c")


@pytest.mark.parametrize("compiler,lang", [("gcc", ["-std=c11"]), ("g++", ["-std=c++17", "-x", "c++"])])
def test_c_consumer_builds_and_passes(tmp_path, compiler, lang):
    assert os.path.exists(os.path.join(LIBDIR, "libengram.so")), "libengram.so not built"
    exe = tmp_path / "abi_consumer"
    subprocess.check_call([compiler, *lang, "-Wall", "-Wextra", "-Werror", "-pedantic",
                           "-I", os.path.join(ROOT, "include"), SRC, "-L", LIBDIR, "-lengram",
                           f"-Wl,-rpath,{LIBDIR}", "-o", str(exe)])
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "abi consumer ok" in r.stdout
