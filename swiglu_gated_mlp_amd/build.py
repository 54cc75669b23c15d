"""Build libswiglu.so (hipcc, gfx950) in-tree, next to this file.

    python -m swiglu_gated_mlp_amd.build

The library is one translation unit: csrc/swiglu_api.hip includes the kernels
from csrc/fused_kernels.hpp and exports the C ABI of include/swiglu.h.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libswiglu.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)
SOURCES = [os.path.join(CSRC, "swiglu_api.hip")]
ARCH = os.environ.get("SWIGLU_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; ROCm is required to build libswiglu")


def compile_flags():
    return [
        "--offload-arch=%s" % ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
        # no packed-fp32 instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC,
    ]


def link_flags():
    # the HIP runtime only: every kernel, the MLP block's down projection
    # included, is this library's own
    return []


def build(verbose: bool = False) -> str:
    """Compile the library (always recompiles) and return its path."""
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *compile_flags(), "-o", tmp, *SOURCES, *link_flags()]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed (%d):\n%s" % (res.returncode, out))
    if verbose and out.strip():
        print(out, flush=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
