"""Build the HIP library libmsda.so in-tree for gfx950 (MI355X)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "msda.hip")
SOURCES = [SRC, os.path.join(PKG, "csrc", "msda3d.hip"), os.path.join(PKG, "csrc", "dat_attn.hip")]
DEPS = SOURCES + [os.path.join(PKG, "csrc", f) for f in ("common.h", "bins.h")]
HEADER = os.path.join(ROOT, "include", "msda.h")
LIB = os.path.join(PKG, "libmsda.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def build(verbose: bool = False, extra=()) -> str:
    cmd = [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-o", LIB + ".tmp",
           *SOURCES]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(f) > t for f in (*DEPS, HEADER))


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
    sys.exit(0)
