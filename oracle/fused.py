"""CPU oracle of the fused prologue (test infrastructure only).

Only ``tests/``, the smoke check and the CPU-baseline leg of ``bench.py`` may
import this module.  It composes the pinned sampling-core oracle
(``msda_oracle.c``) with the two steps that feed it on the first page
("Deformable attention: multi-scale sparse sampling and detection
practice"), written out in plain numpy:

  - section 3.2 (the module's forward): the sampling location is the
    reference point of level l plus the offset divided by that level's
    normalizer (W_l, H_l) -- offsets are in pixels of level l, the location
    is normalized:  loc = ref[b,q,l] + off[b,q,m,l,k] / (W_l, H_l).
    Computed in fp32 (one IEEE division, one addition), the precision the
    GPU library uses, so that both pick the same neighbours.
  - section 3.2 (code) normalizes the attention logits of a (query, head)
    with one softmax over all L*K points; section 2.2 (text) describes a
    softmax over the K points of each level.  Both are offered
    (per_level=False / True).
  - the "Deformable DETR" tutorial, section 3.3 (multi-scale formula): each
    sampled term is weighted by S_qlk * A_qlk, where S_qlk is a separately
    predicted scale attention for level l.  Optional here (scale=None means
    S = 1); when given it is an input of the same shape as the weights,
    [B,Nq,M,L,K], and the core receives the product S * A.

The backward is the chain rule through those steps, in fp64:
grad_offsets = grad_loc / (W_l, H_l); grad_ref[b,q,l] = sum over heads and
points of grad_loc; with g = grad of the product S * A from the core,
grad_scale = A * g and grad_logits = A * (S g - sum_group A * S g) over the
softmax group.
"""
from __future__ import annotations

import numpy as np

import oracle as _core

SPEC = _core.SPEC


def normalizer(spatial_shapes) -> np.ndarray:
    """[L, 2] float32 (W_l, H_l): the divisor of the offsets of level l."""
    s = np.asarray(spatial_shapes, dtype=np.int64)
    return np.stack([s[:, 1], s[:, 0]], axis=-1).astype(np.float32)


def locations(ref, offsets, spatial_shapes) -> np.ndarray:
    """loc[B,Nq,M,L,K,2] float32 = ref[B,Nq,L,2] + offsets / (W_l, H_l), in fp32."""
    ref = np.asarray(ref, dtype=np.float32)
    off = np.asarray(offsets, dtype=np.float32)
    nrm = normalizer(spatial_shapes)
    return (ref[:, :, None, :, None, :] + off / nrm[None, None, None, :, None, :]).astype(
        np.float32)


def weights(logits, L: int, K: int, per_level: bool = False) -> np.ndarray:
    """A[B,Nq,M,L,K] float64: softmax of the logits [B,Nq,M,L*K] over the L*K
    points of a (query, head), or over the K points of each level."""
    z = np.asarray(logits, dtype=np.float64)
    B, Nq, M, LK = z.shape
    assert LK == L * K
    z = z.reshape(B, Nq, M, L, K) if per_level else z.reshape(B, Nq, M, 1, L * K)
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    return (e / e.sum(axis=-1, keepdims=True)).reshape(B, Nq, M, L, K)


def scaled_weights(logits, L: int, K: int, per_level: bool = False, scale=None) -> np.ndarray:
    """S * A [B,Nq,M,L,K] float64: the softmax weights times the scale
    attention (scale=None: S = 1)."""
    A = weights(logits, L, K, per_level)
    return A if scale is None else A * np.asarray(scale, dtype=np.float64)


def forward(value, spatial_shapes, level_start_index, ref, offsets, logits,
            per_level: bool = False, mode: int = SPEC, scale=None) -> np.ndarray:
    """out[B, Nq, M*D] float64 of the core on the fused inputs."""
    L, K = np.asarray(offsets).shape[3], np.asarray(offsets).shape[4]
    loc = locations(ref, offsets, spatial_shapes)
    A = scaled_weights(logits, L, K, per_level, scale).astype(np.float32)
    return _core.forward(value, spatial_shapes, level_start_index, loc, A, mode=mode)


def backward(value, spatial_shapes, level_start_index, ref, offsets, logits, grad_out,
             per_level: bool = False, mode: int = SPEC, scale=None):
    """(grad_value, grad_offsets, grad_logits, grad_ref), float64, and
    grad_scale as a fifth element when scale is given."""
    off = np.asarray(offsets)
    B, Nq, M, L, K, _ = off.shape
    loc = locations(ref, offsets, spatial_shapes)
    A64 = weights(logits, L, K, per_level)
    S64 = np.ones_like(A64) if scale is None else np.asarray(scale, dtype=np.float64)
    gv, gl, ga = _core.backward(value, spatial_shapes, level_start_index, loc,
                               (S64 * A64).astype(np.float32), grad_out, mode=mode)
    nrm = normalizer(spatial_shapes).astype(np.float64)
    g_off = gl / nrm[None, None, None, :, None, :]
    g_ref = gl.sum(axis=(2, 4))                                  # [B, Nq, L, 2]
    gA = S64 * ga                                                # through S * A
    if per_level:
        s = (A64 * gA).sum(axis=-1, keepdims=True)               # per (b, q, m, l)
    else:
        s = (A64 * gA).sum(axis=(-2, -1), keepdims=True)         # per (b, q, m)
    g_logits = (A64 * (gA - s)).reshape(B, Nq, M, L * K)
    if scale is None:
        return gv, g_off, g_logits, g_ref
    return gv, g_off, g_logits, g_ref, A64 * ga
