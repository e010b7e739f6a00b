"""Compile the HIP library ``libsla.so`` for gfx950, in-tree.

Usage: ``python krylov_solvers_adjoint_amd/_build.py`` (always recompiles; run it
by path so that the package, which loads the library, is not imported).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsla.so")
SOURCES = ["api.hip", "csr_build.hip", "cg.hip", "lanczos.hip", "bicgstab.hip", "reorder.hip",
           "noalloc.hip"]
ARCH = os.environ.get("SLA_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # every floating-point * and + is rounded on its own (no fused multiply-add):
    # element-wise results then equal the textbook expression bit for bit
    "-ffp-contract=off",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    # the kernel's first two arguments arrive in scalar registers at wave
    # launch (the solver kernels' only argument is the context pointer):
    # without it the first memory access of every wave waits for a load of
    # that pointer from the argument segment
    "-mllvm", "-amdgpu-kernarg-preload-count=2",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.isabs(cand) and os.path.exists(cand) or not os.path.isabs(cand)):
            return cand
    return "hipcc"


def build(verbose: bool = True) -> str:
    objs = []
    for src in SOURCES:
        obj = os.path.join(CSRC, src.replace(".hip", ".o"))
        cmd = [hipcc(), *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    for o in objs:
        os.remove(o)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
