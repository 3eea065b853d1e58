"""Register and scratch budgets of every HIP kernel, from the compiler's own
resource report (hipcc -Rpass-analysis=kernel-resource-usage) for gfx950.

No kernel may use scratch (private memory) or spill VGPRs (which go to
scratch): a spill would turn register traffic into memory traffic on an
HBM-bound path.  SGPR spills are allowed only where the kernel still has no
scratch: the compiler then keeps them in spare VGPR lanes (a lane write and
read each, no memory).  The gate's backward main
kernel must also keep two waves per SIMD, one 512-thread workgroup per CU,
which its partition of the tokens (all workgroups resident in one round)
assumes.  Compiles the device code only; no GPU is needed."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "memory_bound_engram_amd", "csrc")
SOURCES = ["engram_fwd.hip", "engram_bwd.hip", "engram_gateconv.hip"]

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc not installed")


def _resources():
    flags = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
             "-packed-fp32-ops", "--cuda-device-only", "-c", "-o", os.devnull,
             "-Rpass-analysis=kernel-resource-usage", "-I", os.path.join(ROOT, "include"), "-I", CSRC]
    procs = {src: subprocess.Popen(["hipcc", *flags, os.path.join(CSRC, src)], stdout=subprocess.PIPE,
                                   stderr=subprocess.STDOUT, text=True) for src in SOURCES}
    out = {}
    for src, p in procs.items():
        text, _ = p.communicate(timeout=900)
        assert p.returncode == 0, text[-2000:]
        kernels = {}
        name = None
        for line in text.splitlines():
            m = re.search(r"Function Name: (\S+)", line)
            if m:
                name = m.group(1)
                kernels[name] = {}
                continue
            m = re.search(r"remark:\s+([A-Za-z][A-Za-z /\[\]]*?):\s+(-?\d+)", line)
            if m and name:
                kernels[name][m.group(1).strip()] = int(m.group(2))
        out[src] = kernels
    return out


@pytest.fixture(scope="module")
def resources():
    return _resources()


def test_every_kernel_is_reported(resources):
    for src in SOURCES:
        assert resources[src], f"no kernels reported for {src}"
    names = " ".join(k for r in resources.values() for k in r)
    for k in ("engram_fwd_kernel", "engram_fwd_paced_kernel", "engram_bwd_main_kernel", "engram_bwd_reduce_kernel",
              "gateconv_fwd_kernel", "gateconv_bwd_conv_kernel", "gateconv_bwd_hk_kernel", "gateconv_reduce_kernel"):
        assert k in names, k


def test_no_kernel_uses_scratch(resources):
    keys = ("ScratchSize [bytes/lane]", "VGPRs Spill", "SGPRs Spill")
    for rs in resources.values():
        for r in rs.values():
            assert all(k in r for k in keys), r  # the report format is the one parsed here
    spills = {k: {x: r[x] for x in keys} for rs in resources.values() for k, r in rs.items()
              if r["ScratchSize [bytes/lane]"] != 0 or r["VGPRs Spill"] != 0}
    assert not spills, spills


def test_backward_main_kernel_occupancy(resources):
    (main,) = [r for k, r in resources["engram_bwd.hip"].items() if "engram_bwd_main_kernel" in k]
    assert main["Occupancy [waves/SIMD]"] >= 2, main
    assert main["VGPRs"] <= 256, main


def test_gateconv_backward_occupancy(resources):
    """The GateConv chunk rule sizes the backward's grid for the workgroups a
    CU holds at once: two of the conv kernel's 4-wave workgroups at d = 2560
    (256 x 10 map) and two of its 12-wave ones at d = 1536 (768 x 2 map), and
    one 8-wave workgroup at d = 5120.  Occupancy here is waves per SIMD (a CU
    has four SIMDs), so those need 2, 6 and 2 waves per SIMD."""
    conv = {k: r for k, r in resources["engram_gateconv.hip"].items() if "gateconv_bwd_conv_kernel" in k}
    want = {"ColMapILi256ELi10E": 2, "ColMapILi768ELi2E": 6, "ColMapILi512ELi10E": 2}
    for tag, waves in want.items():
        (r,) = [r for k, r in conv.items() if tag in k]
        assert r["Occupancy [waves/SIMD]"] >= waves, (tag, r)
