"""CPU oracle of the 3-D (trilinear) sampling core (test infrastructure only).

Only ``tests/``, the smoke check and the CPU-baseline leg of ``bench.py`` may
import this module.  It wraps ``msda3d_oracle.c`` (plain loops, fp64
accumulation) through ctypes; the computation -- the first page's section 5.3
variant for voxel features, the 2-D core with a third coordinate and eight
trilinear neighbours -- is documented in that file's header.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

import oracle as _core

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "msda3d_oracle.c")
LIB_PATH = os.path.join(_HERE, "libmsda3d_oracle.so")
SPEC, DOUBLE, ALIGN = _core.SPEC, _core.DOUBLE, _core.ALIGN
_default = None


def build(verbose: bool = False, src: str = SRC, out: str = LIB_PATH, extra=()) -> str:
    return _core.build(verbose=verbose, src=src, out=out, extra=extra)


class VolumeLib:
    """ctypes handle on one compiled copy of msda3d_oracle.c."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        p, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.oracle3d_forward.argtypes = [p] * 6 + [i64] * 7 + [ci, ci]
        lib.oracle3d_forward.restype = ci
        lib.oracle3d_backward.argtypes = [p] * 9 + [i64] * 7 + [ci, ci]
        lib.oracle3d_backward.restype = ci
        self.lib = lib

    def forward(self, value, shapes, starts, loc, attn, mode=SPEC, threads=0):
        """out[B, Nq, M*D] (float64)."""
        value, loc, attn = _f32(value), _f32(loc), _f32(attn)
        shapes, starts = _i64(shapes).reshape(-1, 3), _i64(starts)
        B, Nv, Nq, M, D, L, K = _dims(value, shapes, loc, attn)
        out = np.zeros((B, Nq, M * D), dtype=np.float64)
        rc = self.lib.oracle3d_forward(_ptr(value), _ptr(shapes), _ptr(starts), _ptr(loc),
                                       _ptr(attn), _ptr(out), B, Nv, Nq, M, D, L, K,
                                       int(mode), int(threads))
        if rc != 0:
            raise ValueError(f"oracle3d_forward rejected its arguments (code {rc})")
        return out

    def backward(self, value, shapes, starts, loc, attn, grad_out, mode=SPEC, threads=0):
        """(grad_value, grad_sampling_loc, grad_attn_weight), float64."""
        value, loc, attn = _f32(value), _f32(loc), _f32(attn)
        shapes, starts = _i64(shapes).reshape(-1, 3), _i64(starts)
        B, Nv, Nq, M, D, L, K = _dims(value, shapes, loc, attn)
        g = _f32(grad_out).reshape(B, Nq, M * D)
        gv = np.zeros((B, Nv, M, D), dtype=np.float64)
        gl = np.zeros((B, Nq, M, L, K, 3), dtype=np.float64)
        ga = np.zeros((B, Nq, M, L, K), dtype=np.float64)
        rc = self.lib.oracle3d_backward(_ptr(value), _ptr(shapes), _ptr(starts), _ptr(loc),
                                        _ptr(attn), _ptr(g), _ptr(gv), _ptr(gl), _ptr(ga),
                                        B, Nv, Nq, M, D, L, K, int(mode), int(threads))
        if rc != 0:
            raise ValueError(f"oracle3d_backward rejected its arguments (code {rc})")
        return gv, gl, ga


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _i64(a):
    return np.ascontiguousarray(a, dtype=np.int64)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dims(value, shapes, loc, attn):
    B, Nv, M, D = value.shape
    L = shapes.shape[0]
    Bq, Nq, Mq, Lq, K, three = loc.shape
    if (Bq, Mq, Lq, three) != (B, M, L, 3):
        raise ValueError(f"sampling_loc shape {loc.shape} does not match value {value.shape}"
                         f" and {L} levels")
    if attn.shape != (B, Nq, M, L, K):
        raise ValueError(f"attn_weight shape {attn.shape} != {(B, Nq, M, L, K)}")
    return B, Nv, Nq, M, D, L, K


def default() -> VolumeLib:
    """The oracle built from oracle/msda3d_oracle.c (compiled on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC):
            build()
        _default = VolumeLib(LIB_PATH)
    return _default


def forward(*args, **kw):
    return default().forward(*args, **kw)


def backward(*args, **kw):
    return default().backward(*args, **kw)
