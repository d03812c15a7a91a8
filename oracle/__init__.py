"""CPU oracle for the MSDeformAttn sampling core (test infrastructure only).

Only ``tests/``, the smoke check and the CPU-baseline leg of ``bench.py`` may
import this package.  It wraps ``msda_oracle.c`` (plain loops, fp64
accumulation) through ctypes and shares nothing with the GPU library.

The computation it follows is documented in the header of ``msda_oracle.c``:
the multi-scale formula of "Deformable attention: multi-scale sparse sampling
and detection practice" section 2.2, its bilinear tent weights with zero
padding (section 2.3) and the align_corners=False pixel mapping of its
grid_sample module (sections 2.3 and 3.2).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msda_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmsda_oracle.so")
_default = None

SPEC = 0    # fp32 coordinate transform (fmaf + floorf), as the GPU library does
DOUBLE = 1  # every coordinate step in fp64
ALIGN = 2   # flag: x = u*(W-1), y = v*(H-1) (align_corners=True); combine with SPEC/DOUBLE


def build(verbose: bool = False, src: str = _SRC, out: str = _LIB_PATH, extra=()) -> str:
    """Compile the oracle with gcc (-O2, no FMA contraction, OpenMP); extra
    flags are appended (the CPU sanitizer build passes its own)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
           "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra", *extra, "-o",
           out + ".tmp", src, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class OracleLib:
    """ctypes handle on one compiled copy of msda_oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        ci = ctypes.c_int
        lib.oracle_forward.argtypes = [p, p, p, p, p, p] + [i64] * 7 + [ci, ci]
        lib.oracle_forward.restype = ci
        lib.oracle_backward.argtypes = [p] * 9 + [i64] * 7 + [ci, ci]
        lib.oracle_backward.restype = ci
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ci
        self.lib = lib
        self.path = path

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    def forward(self, *args, **kw):
        return _forward(self.lib, *args, **kw)

    def backward(self, *args, **kw):
        return _backward(self.lib, *args, **kw)


def default() -> OracleLib:
    """The oracle built from oracle/msda_oracle.c (compiled on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB_PATH) or (
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
            build()
        _default = OracleLib(_LIB_PATH)
    return _default


def _load():
    return default().lib


def max_threads() -> int:
    return default().max_threads()


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i64(a):
    return np.ascontiguousarray(a, dtype=np.int64)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dims(value, shapes, loc):
    B, Nv, M, D = value.shape
    L = shapes.shape[0]
    Bq, Nq, Mq, Lq, K, two = loc.shape
    if (Bq, Mq, Lq, two) != (B, M, L, 2):
        raise ValueError(f"sampling_loc shape {loc.shape} does not match value {value.shape}"
                         f" and {L} levels")
    return B, Nv, Nq, M, D, L, K


def forward(*args, **kw) -> np.ndarray:
    """out[B, Nq, M*D] (float64); see _forward."""
    return _forward(_load(), *args, **kw)


def backward(*args, **kw):
    """(grad_value, grad_sampling_loc, grad_attn_weight) as float64; see _backward."""
    return _backward(_load(), *args, **kw)


def _forward(lib, value, spatial_shapes, level_start_index, sampling_loc, attn_weight,
             mode: int = SPEC, threads: int = 0) -> np.ndarray:
    """out[B, Nq, M*D] (float64) for the given inputs (see msda_oracle.c)."""
    value, loc, attn = _f32(value), _f32(sampling_loc), _f32(attn_weight)
    shapes, start = _i64(spatial_shapes), _i64(level_start_index)
    B, Nv, Nq, M, D, L, K = _dims(value, shapes, loc)
    if attn.shape != (B, Nq, M, L, K):
        raise ValueError(f"attn_weight shape {attn.shape} != {(B, Nq, M, L, K)}")
    out = np.zeros((B, Nq, M * D), dtype=np.float64)
    rc = lib.oracle_forward(_ptr(value), _ptr(shapes), _ptr(start), _ptr(loc),
                            _ptr(attn), _ptr(out), B, Nv, Nq, M, D, L, K,
                            int(mode), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_forward rejected its arguments (code {rc})")
    return out


def _backward(lib, value, spatial_shapes, level_start_index, sampling_loc, attn_weight,
              grad_out, mode: int = SPEC, threads: int = 0):
    """(grad_value, grad_sampling_loc, grad_attn_weight) as float64 arrays."""
    value, loc, attn = _f32(value), _f32(sampling_loc), _f32(attn_weight)
    shapes, start = _i64(spatial_shapes), _i64(level_start_index)
    B, Nv, Nq, M, D, L, K = _dims(value, shapes, loc)
    g = _f32(grad_out).reshape(B, Nq, M * D)
    gv = np.zeros((B, Nv, M, D), dtype=np.float64)
    gl = np.zeros((B, Nq, M, L, K, 2), dtype=np.float64)
    ga = np.zeros((B, Nq, M, L, K), dtype=np.float64)
    rc = lib.oracle_backward(_ptr(value), _ptr(shapes), _ptr(start), _ptr(loc),
                             _ptr(attn), _ptr(g), _ptr(gv), _ptr(gl), _ptr(ga),
                             B, Nv, Nq, M, D, L, K, int(mode), int(threads))
    if rc != 0:
        raise ValueError(f"oracle_backward rejected its arguments (code {rc})")
    return gv, gl, ga
