"""Builds libgenrec.so (HIP, gfx950) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libgenrec.so")
SOURCES = ["kernels.hip", "api.cpp"]
ARCH = os.environ.get("GENREC_ARCH", "gfx950")

# Packed-fp32 instructions are kept out of the generated code on purpose.
HIP_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument"]


def build(verbose: bool = False) -> str:
    objs = []
    bdir = os.path.join(PKG, "_build")
    os.makedirs(bdir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        cmd = ["hipcc", *HIP_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), file=sys.stderr)
        subprocess.check_call(cmd, stderr=None if verbose else subprocess.DEVNULL
                              if os.environ.get("GENREC_QUIET_BUILD") else None)
        objs.append(obj)
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.check_call(["hipcc", "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
