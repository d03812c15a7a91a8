"""Build the HIP libraries in-tree for gfx950 (MI355X): libmsda.so (the
sampling core and its C ABI) and libmsda_probe.so (measurement kernels the
benchmark uses for the roofline).  Sources are compiled in parallel, then
linked.  The host-only part of the C ABI (csrc/host_checks.cpp) is compiled
by the host compiler; build_host_sanitized() builds it alone with the
address and undefined-behaviour sanitizers for the CPU tests."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("msda.hip", "msda3d.hip", "dat_attn.hip")]
PROBE_SOURCES = [os.path.join(CSRC, "probe.hip")]
HOST_SOURCE = os.path.join(CSRC, "host_checks.cpp")
DEPS = SOURCES + [HOST_SOURCE] + [os.path.join(CSRC, f)
                                  for f in ("common.h", "bins.h", "host_checks.h")]
HEADER = os.path.join(ROOT, "include", "msda.h")
LIB = os.path.join(PKG, "libmsda.so")
PROBE_LIB = os.path.join(PKG, "libmsda_probe.so")
OBJ_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CXX = os.environ.get("CXX", "g++")
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]
SANITIZED_HOST_LIB = os.path.join(OBJ_DIR, "libmsda_host_sanitized.so")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
]


def _objects(sources, verbose, extra):
    os.makedirs(OBJ_DIR, exist_ok=True)
    procs, objs = [], []
    for src in sources:
        obj = os.path.join(OBJ_DIR, os.path.basename(src) + ".o")
        if src.endswith(".cpp"):
            cmd = [CXX, *HOST_FLAGS, "-I", os.path.join(ROOT, "include"), "-c", "-o", obj, src]
        else:
            cmd = [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c", "-o", obj,
                   src]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), cmd))
        objs.append(obj)
    for p, cmd in procs:
        if p.wait() != 0:
            raise subprocess.CalledProcessError(p.returncode, cmd)
    return objs


def _link(objs, out, verbose):
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", out + ".tmp", *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)


def build(verbose: bool = False, extra=()) -> str:
    objs = _objects(SOURCES + [HOST_SOURCE] + PROBE_SOURCES, verbose, extra)
    _link(objs[:len(SOURCES) + 1], LIB, verbose)
    _link(objs[len(SOURCES) + 1:], PROBE_LIB, verbose)
    return LIB


def build_host_sanitized(verbose: bool = False) -> str:
    """host_checks.cpp alone, with the address and undefined-behaviour
    sanitizers (host code only: no GPU code is involved), into
    _build/libmsda_host_sanitized.so."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    out = SANITIZED_HOST_LIB
    cmd = [CXX, "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-o", out + ".tmp", HOST_SOURCE]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def stale() -> bool:
    if not (os.path.exists(LIB) and os.path.exists(PROBE_LIB)):
        return True
    t = min(os.path.getmtime(LIB), os.path.getmtime(PROBE_LIB))
    return any(os.path.getmtime(f) > t for f in (*DEPS, *PROBE_SOURCES, HEADER))


if __name__ == "__main__":
    build(verbose=True)
    print(LIB)
    print(PROBE_LIB)
    sys.exit(0)
