"""Build libengram.so (the HIP kernels and the C ABI) for gfx950 with hipcc."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libengram.so")

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    # no packed-fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]
    if r.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc failed ({r.returncode}) building {LIB}")
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIB)
    return LIB


PROBE_SRC = os.path.join(PKG, "probe", "hbm_probe.hip")
PROBE_BIN = os.path.join(PKG, "probe", "hbm_probe")
VALU_SRC = os.path.join(PKG, "probe", "valu_rate.hip")
VALU_BIN = os.path.join(PKG, "probe", "valu_rate")


def _build_program(src: str, out: str) -> str:
    tmp = out + ".tmp"
    cmd = ["hipcc", *[f for f in HIPCC_FLAGS if f not in ("-fPIC", "-shared")], "-o", tmp, src]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode}) building {out}")
    os.replace(tmp, out)
    return out


def build_probe(verbose: bool = False) -> str:
    """The measurement programs (not part of libengram): the HBM streaming
    ceilings (hbm_probe) and the VALU issue costs (valu_rate)."""
    _build_program(VALU_SRC, VALU_BIN)
    return _build_program(PROBE_SRC, PROBE_BIN)


PROBE_LIB_SRC = os.path.join(PKG, "probe", "stream_lib.hip")
PROBE_LIB = os.path.join(PKG, "probe", "libengram_probe.so")


def build_probe_lib(verbose: bool = False) -> str:
    """The probe's streaming kernels as a shared library (bench.py --same-buffers)."""
    tmp = PROBE_LIB + ".tmp"
    cmd = ["hipcc", *HIPCC_FLAGS, "-o", tmp, PROBE_LIB_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode}) building {PROBE_LIB}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_probe(verbose=True))
    print(build_probe_lib(verbose=True))
