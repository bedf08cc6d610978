"""Build libmoe_ep.so (the C-ABI HIP library) in-tree with hipcc for gfx950.

    python combine_moe_dispatch_amd/_build.py

(run as a file, not as a module of the package: importing the package loads
the library this script builds)

Flags: -O3; packed fp32 instructions disabled (-packed-fp32-ops); fp32 divide
correctly rounded (the fp8 block scales depend on it); no fast-math.  Links
the ROCTX library of the ROCm install (ranges around the four calls).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "lib")
LIB_PATH = os.path.join(LIB_DIR, "libmoe_ep.so")
SOURCES = [os.path.join(CSRC, "moe_ep.hip"), os.path.join(CSRC, "moe_kernels.hip")]
ARCH = "gfx950"


def rocm() -> str:
    return os.environ.get("ROCM_PATH", "/opt/rocm")


def hipcc() -> str:
    cand = os.path.join(rocm(), "bin", "hipcc")
    return cand if os.path.exists(cand) else "hipcc"


def build(verbose: bool = False) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Wall", "-Wno-unused-result",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-fast-math",
           "-I", INCLUDE, "-I", CSRC, "-o", tmp] + SOURCES + [
           # ROCTX ranges around the four calls (rocprofv3 --marker-trace)
           "-L", os.path.join(rocm(), "lib"), "-lrocprofiler-sdk-roctx",
           "-Wl,-rpath," + os.path.join(rocm(), "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
