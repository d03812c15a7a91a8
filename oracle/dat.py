"""CPU oracle of DAT's sampled-key attention (test infrastructure only).

Only ``tests/``, the smoke check and the CPU-baseline leg of ``bench.py`` may
import this module.  What it follows -- the DAT integration page (the
`DAttentionBaseline` walk-through, sections 2.1 to 2.3) and the first page's
section 5.1:

  - section 2.1/2.2: a reference grid of Hk x Wk points (one per r x r cell of
    the H x W feature map) is moved by predicted offsets, and the features
    are sampled there with bilinear grid_sample, align_corners=True, zero
    padding, per group of C/G channels (G offset groups).  With the features
    channel-last as value [B, H*W, G, C/G] and the positions as normalized
    (u, v) in [0, 1] this is the sampling core with one level, one point per
    sampled key, weight 1 and the align-corners convention: ``sample`` calls
    the (pinned) core oracle that way.
  - section 2.3: the keys and values (projections of the sampled features,
    outside this path) enter standard multi-head attention with the queries:
    per batch b and head h, S = scale * Q K^T + bias (the deformable
    relative-position bias; its construction is elided on the page, so it is
    an optional input here), P = softmax of S over the Ns keys, O = P V.
    ``attention`` writes that out in fp64 with numpy.

The backward is the chain rule, in fp64:
    dP = dO V^T,  dS = P * (dP - rowsum(P * dP)),
    dQ = scale * dS K,  dK = scale * dS^T Q,  dV = P^T dO,  dbias = dS.

Layouts (channel-last, as the GPU library):
    q      [B, N, Hh, d]     k, v  [B, Ns, Hh, d]     bias [B, Hh, N, Ns]
    out    [B, N, Hh, d]     lse   [B, Hh, N]  (log-sum-exp of each row of S)
"""
from __future__ import annotations

import numpy as np

import oracle as _core


def sample(value, hw, pos, mode=_core.SPEC):
    """Sampled features [B, Ns, G*Dg] (float64): value [B, H*W, G, Dg],
    hw = (H, W), pos [B, Ns, G, 2] normalized (u, v) along (x, y)."""
    H, W = (int(v) for v in hw)
    value = np.asarray(value, dtype=np.float32)
    B, Nv, G, Dg = value.shape
    pos = np.asarray(pos, dtype=np.float32)
    Ns = pos.shape[1]
    loc = pos.reshape(B, Ns, G, 1, 1, 2)
    ones = np.ones((B, Ns, G, 1, 1), np.float32)
    return _core.forward(value, np.array([[H, W]], np.int64), np.zeros(1, np.int64), loc, ones,
                         mode=mode | _core.ALIGN)


def sample_backward(value, hw, pos, grad_sampled, mode=_core.SPEC):
    """(grad_value [B, H*W, G, Dg], grad_pos [B, Ns, G, 2]) as float64."""
    H, W = (int(v) for v in hw)
    value = np.asarray(value, dtype=np.float32)
    B, Nv, G, Dg = value.shape
    pos = np.asarray(pos, dtype=np.float32)
    Ns = pos.shape[1]
    loc = pos.reshape(B, Ns, G, 1, 1, 2)
    ones = np.ones((B, Ns, G, 1, 1), np.float32)
    gv, gl, _ = _core.backward(value, np.array([[H, W]], np.int64), np.zeros(1, np.int64), loc,
                               ones, grad_sampled, mode=mode | _core.ALIGN)
    return gv, gl.reshape(B, Ns, G, 2)


def _scores(q, k, bias, scale):
    s = scale * np.einsum("bnhd,bshd->bhns", q, k)
    if bias is not None:
        s = s + np.asarray(bias, dtype=np.float64)
    return s


def attention(q, k, v, bias=None, scale=None):
    """(out [B, N, Hh, d], lse [B, Hh, N]) in float64."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    if scale is None:
        scale = q.shape[-1] ** -0.5
    s = _scores(q, k, bias, scale)
    mx = s.max(axis=-1, keepdims=True)
    e = np.exp(s - mx)
    tot = e.sum(axis=-1, keepdims=True)
    p = e / tot
    out = np.einsum("bhns,bshd->bnhd", p, v)
    lse = (mx + np.log(tot))[..., 0]
    return out, lse


def attention_backward(q, k, v, grad_out, bias=None, scale=None):
    """(dq, dk, dv, dbias) in float64."""
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    g = np.asarray(grad_out, dtype=np.float64)
    if scale is None:
        scale = q.shape[-1] ** -0.5
    s = _scores(q, k, bias, scale)
    e = np.exp(s - s.max(axis=-1, keepdims=True))
    p = e / e.sum(axis=-1, keepdims=True)
    dp = np.einsum("bnhd,bshd->bhns", g, v)
    ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))
    dq = scale * np.einsum("bhns,bshd->bnhd", ds, k)
    dk = scale * np.einsum("bhns,bnhd->bshd", ds, q)
    dv = np.einsum("bhns,bnhd->bshd", p, g)
    return dq, dk, dv, ds
