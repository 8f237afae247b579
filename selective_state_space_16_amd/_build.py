"""Compile libssm.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libssm.so")
CALIB_LIB = os.path.join(PKG, "libssm_calib.so")
CALIB_SOURCE = "ssm_calib.hip"
ARCH = os.environ.get("SSM_OFFLOAD_ARCH", "gfx950")

SOURCES = ["ssm_scan_stripe_act.hip", "ssm_scan_stripe_conv.hip", "ssm_scan_stripe_trap.hip", "ssm_scan_stripe.hip", "ssm_scan.hip", "ssm_step.hip", "ssm_ssd.hip", "ssm_ssd_step.hip", "ssm_scan_bwd_trap.hip", "ssm_scan_bwd.hip", "ssm_conv_bwd.hip", "ssm_noalloc.hip", "ssm_abi.cpp"]

# -packed-fp32-ops keeps the compiler from emitting packed fp32 VALU forms.
# The atomic optimizer is off: it rewrites a one-lane atomic with a returned
# value into a wave-wide pattern that waits for the result right away, and the
# scan's tile counter is read only at the end of a tile.
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-ffp-contract=fast", "-Wall", "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(out: str = LIB, verbose: bool = False) -> str:
    """Compile every source into one shared library (always rebuilds). The
    sources compile in parallel; the two tiled-scan files take the longest."""
    from concurrent.futures import ThreadPoolExecutor
    tmpdir = os.path.join(PKG, "_build")
    os.makedirs(tmpdir, exist_ok=True)
    cc = hipcc()

    def compile_one(src):
        path = os.path.join(CSRC, src)
        obj = os.path.join(tmpdir, src + ".o")
        cmd = [cc] + HIP_FLAGS + ["-I", os.path.join(ROOT, "include"), "-c", path, "-o", obj]
        if src.endswith(".cpp"):
            cmd = [cc, "-O2", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include"),
                   "-c", path, "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.run(cmd, check=True)
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES) + 1, os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES + [CALIB_SOURCE]))
    calib_obj = objs.pop()
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    # the issue-rate calibration kernels, a library of their own (bench.py
    # --valu-calibration); libssm does not contain or load them
    tmp = CALIB_LIB + ".tmp%d" % os.getpid()
    cmd = [cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, calib_obj]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, CALIB_LIB)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
