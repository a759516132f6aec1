"""Build the gfx950 shared library libnvfp4gg.so in-tree with hipcc.

Usage: python precision_moe_nvfp4_amd/build.py [-v]   (run as a script: importing it through
the package would first load the library it builds)
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libnvfp4gg.so")
SOURCES = ["nvfp4_gg_kernels.hip", "nvfp4_gg_api.cpp"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU instructions.
FLAGS = [
    "--offload-arch=gfx950", "-mcode-object-version=5", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-Wno-unused-command-line-argument",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    srcs = []
    for s in SOURCES:
        path = os.path.join(CSRC, s)
        if s.endswith(".cpp"):
            srcs += ["-x", "hip", path]
        else:
            srcs.append(path)
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
