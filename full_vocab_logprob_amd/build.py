"""Build libflare_logprobs.so for gfx950 with hipcc (in-tree).

The kernels are compiled with FP contraction off (the reported value must be
a plain FP32 subtraction) and with packed-FP32 instructions disabled.
"""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libflare_logprobs.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", "-ffp-contract=off", "-Wall",
          "-I", os.path.join(ROOT, "include")]
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    kobj = os.path.join(LIBDIR, "flp_kernels.o")
    hobj = os.path.join(LIBDIR, "flp_host.o")
    cmds = [
        [HIPCC, *COMMON, *DEVICE, "-x", "hip", "-c", os.path.join(CSRC, "flp_kernels.hip"),
         "-o", kobj],
        [HIPCC, *COMMON, f"--offload-arch={ARCH}", "-c", os.path.join(CSRC, "flp_host.cpp"),
         "-o", hobj],
        [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", kobj, hobj, "-o", LIB + ".tmp"],
    ]
    for c in cmds:
        if verbose:
            print(" ".join(c))
        subprocess.run(c, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
