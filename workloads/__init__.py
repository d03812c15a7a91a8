"""Seeded synthetic inputs for the MSDeformAttn sampling core.

This module only draws inputs; it holds none of the sampling arithmetic.  The
tests, the smoke check and the benchmark take their inputs from here, and the
same arrays go to the GPU library and to the CPU oracle.

Shapes follow the workloads the pages describe:
  * "Deformable attention: multi-scale sparse sampling and detection
    practice", section 1.1: an 800x1333 image gives four levels at strides
    8..64 of 100x167, 50x84, 25x42 and 13x21 pixels (22,223 tokens), and every
    flattened pixel is an encoder query; K=4 points per level, 8 heads,
    d_model 256 (so 32 channels per head), section 2.2 and the module of 3.2.
  * "Deformable DETR" tutorial, section 4.3: the decoder uses 300 object
    queries that sample the encoder memory.
  * the dense-point variant with K=8 (first page, sections 2.1 and 4.3).
No dataset is read: random normal features stand in for backbone features and
random references/offsets for learned ones.

Random numbers: numpy Generator(PCG64(seed)) with seed = 1000*config + tensor
id (0 value, 1 reference, 2 offsets, 3 logits, 4 grad_out, 5 direct
locations, 6 scale attention).  Draws are float64 and rounded to float32 with round-to-nearest-
even; bfloat16 values are round-to-nearest-even from those float32 values.
Attention weights are a softmax over the L*K logits of one (query, head), as
in the first page's module (section 3.2); locations are reference + offset,
with offsets drawn in pixels of each level and divided by that level's
(W, H), as in the tutorial's pseudocode (section 6).
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional, Sequence, Tuple

import numpy as np

DETR_LEVELS: Tuple[Tuple[int, int], ...] = ((100, 167), (50, 84), (25, 42), (13, 21))

CONFIG_NAMES = ("tiny", "encoder", "decoder", "encoder_bwd", "train_bf16")


def level_table(shapes: Sequence[Tuple[int, int]]):
    """(spatial_shapes int64 [L,2] rows (H,W), level_start_index int64 [L])."""
    ss = np.asarray(shapes, dtype=np.int64).reshape(-1, 2)
    sizes = ss[:, 0] * ss[:, 1]
    start = np.zeros(len(ss), dtype=np.int64)
    if len(ss) > 1:
        start[1:] = np.cumsum(sizes)[:-1]
    return ss, start


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def softmax_lastaxis(logits: np.ndarray) -> np.ndarray:
    z = logits - logits.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


@dataclasses.dataclass
class Workload:
    name: str
    value: np.ndarray                 # [B,Nv,M,D] float32 (bf16-rounded when value_bf16 is set)
    spatial_shapes: np.ndarray        # [L,2] int64 rows (H,W)
    level_start_index: np.ndarray     # [L] int64
    sampling_loc: np.ndarray          # [B,Nq,M,L,K,2] float32
    attn_weight: np.ndarray           # [B,Nq,M,L,K] float32
    grad_out: Optional[np.ndarray]    # [B,Nq,M*D] float32
    value_bf16: Optional[np.ndarray] = None   # [B,Nv,M,D] uint16 bits
    value_unrounded: Optional[np.ndarray] = None  # float32 before bf16 rounding

    @property
    def dims(self):
        B, Nv, M, D = self.value.shape
        _, Nq, _, L, K, _ = self.sampling_loc.shape
        return dict(B=B, Nv=Nv, Nq=Nq, M=M, D=D, L=L, K=K)

    @property
    def points(self) -> int:
        d = self.dims
        return d["B"] * d["Nq"] * d["M"] * d["L"] * d["K"]

    def sha256(self) -> dict:
        """SHA-256 of each input array's bytes (C order), by field name."""
        out = {}
        for f in ("value", "sampling_loc", "attn_weight", "grad_out", "value_bf16"):
            a = getattr(self, f)
            if a is not None:
                out[f] = hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
        return out


def _weights(seed: int, B: int, Nq: int, M: int, L: int, K: int) -> np.ndarray:
    logits = _rng(seed).standard_normal((B, Nq, M, L * K))
    return softmax_lastaxis(logits).reshape(B, Nq, M, L, K).astype(np.float32)


def _encoder_refs(shapes) -> np.ndarray:
    """Normalized pixel centre of every flattened pixel, in its own level: [Nv, 2] (x, y)."""
    refs = []
    for H, W in shapes:
        ys, xs = np.meshgrid((np.arange(H) + 0.5) / H, (np.arange(W) + 0.5) / W, indexing="ij")
        refs.append(np.stack([xs.ravel(), ys.ravel()], axis=-1))
    return np.concatenate(refs, axis=0)


def _locations(ref_bq2: np.ndarray, seed: int, M: int, shapes, K: int, sigma_px: float):
    """ref [B,Nq,2] shared over heads and levels; offsets N(0, sigma px)/(W_l, H_l)."""
    B, Nq, _ = ref_bq2.shape
    L = len(shapes)
    off = _rng(seed).standard_normal((B, Nq, M, L, K, 2)) * sigma_px
    wh = np.array([[w, h] for (h, w) in shapes], dtype=np.float64)  # [L,2] (W,H)
    loc = ref_bq2[:, :, None, None, None, :] + off / wh[None, None, None, :, None, :]
    return loc.astype(np.float32)


def make(config: int | str, batch: Optional[int] = None) -> Workload:
    """Build one of the five configurations (by index 0..4 or name)."""
    idx = CONFIG_NAMES.index(config) if isinstance(config, str) else int(config)
    name = CONFIG_NAMES[idx]
    base = 1000 * idx
    if idx == 0:
        shapes = ((8, 8), (4, 4))
        B, M, D, K, Nq = 1, 2, 8, 2, 16
        ss, st = level_table(shapes)
        Nv = int(ss.prod(axis=1).sum())
        L = len(shapes)
        value = _rng(base + 0).standard_normal((B, Nv, M, D)).astype(np.float32)
        loc = _rng(base + 5).uniform(-0.1, 1.1, (B, Nq, M, L, K, 2)).astype(np.float32)
        w = _weights(base + 3, B, Nq, M, L, K)
        g = _rng(base + 4).standard_normal((B, Nq, M * D)).astype(np.float32)
        return Workload(name, value, ss, st, loc, w, g)

    shapes = DETR_LEVELS
    ss, st = level_table(shapes)
    Nv = int(ss.prod(axis=1).sum())
    L = len(shapes)
    M, D = 8, 32
    if idx in (1, 3):
        B, K, Nq, sigma = 2, 4, Nv, 2.0
    elif idx == 2:
        B, K, Nq, sigma = 2, 4, 300, 4.0
    else:
        B, K, Nq, sigma = 4, 8, Nv, 3.0
    if batch is not None:
        B = int(batch)
    vals = _rng(base + 0).standard_normal((B, Nv, M, D)).astype(np.float32)
    if idx == 2:
        ref = _rng(base + 1).uniform(0.05, 0.95, (B, Nq, 2))
    else:
        ref = np.broadcast_to(_encoder_refs(shapes)[None], (B, Nq, 2))
    loc = _locations(ref, base + 2, M, shapes, K, sigma)
    w = _weights(base + 3, B, Nq, M, L, K)
    g = None
    if idx in (2, 3, 4):
        g = _rng(base + 4).standard_normal((B, Nq, M * D)).astype(np.float32)
    if idx == 4:
        bits = bf16_bits(vals)
        return Workload(name, bf16_to_f32(bits).reshape(vals.shape), ss, st, loc, w, g,
                        value_bf16=bits.reshape(vals.shape), value_unrounded=vals)
    return Workload(name, vals, ss, st, loc, w, g)


def random_case(seed: int, B: int, shapes, Nq: int, M: int, D: int, K: int,
                loc_low: float = -0.1, loc_high: float = 1.1, bf16: bool = False,
                with_grad: bool = True) -> Workload:
    """Small random case: iid uniform locations in [loc_low, loc_high)."""
    ss, st = level_table(shapes)
    Nv = int(ss.prod(axis=1).sum()) if len(shapes) else 0
    L = len(shapes)
    r = _rng(seed)
    vals = r.standard_normal((B, Nv, M, D)).astype(np.float32)
    loc = r.uniform(loc_low, loc_high, (B, Nq, M, L, K, 2)).astype(np.float32)
    logits = r.standard_normal((B, Nq, M, L * K))
    w = softmax_lastaxis(logits).reshape(B, Nq, M, L, K).astype(np.float32) if L * K else \
        np.zeros((B, Nq, M, L, K), np.float32)
    g = r.standard_normal((B, Nq, M * D)).astype(np.float32) if with_grad else None
    name = f"random(seed={seed})"
    if bf16:
        bits = bf16_bits(vals)
        return Workload(name, bf16_to_f32(bits).reshape(vals.shape), ss, st, loc, w, g,
                        value_bf16=bits.reshape(vals.shape), value_unrounded=vals)
    return Workload(name, vals, ss, st, loc, w, g)


@dataclasses.dataclass
class FusedWorkload:
    """Inputs of the fused prologue: raw offsets and logits plus reference points."""
    name: str
    value: np.ndarray                 # [B,Nv,M,D] float32 (bf16-rounded when value_bf16 is set)
    spatial_shapes: np.ndarray        # [L,2] int64 rows (H,W)
    level_start_index: np.ndarray     # [L] int64
    reference_points: np.ndarray      # [B,Nq,L,2] float32, normalized (x, y)
    sampling_offsets: np.ndarray      # [B,Nq,M,L,K,2] float32, pixels of level l
    attn_logits: np.ndarray           # [B,Nq,M,L*K] float32
    grad_out: Optional[np.ndarray]    # [B,Nq,M*D] float32
    value_bf16: Optional[np.ndarray] = None   # [B,Nv,M,D] uint16 bits
    attn_scale: Optional[np.ndarray] = None   # [B,Nq,M,L,K] float32 scale attention S

    @property
    def dims(self):
        B, Nv, M, D = self.value.shape
        _, Nq, _, L, K, _ = self.sampling_offsets.shape
        return dict(B=B, Nv=Nv, Nq=Nq, M=M, D=D, L=L, K=K)

    @property
    def points(self) -> int:
        d = self.dims
        return d["B"] * d["Nq"] * d["M"] * d["L"] * d["K"]


def scale_attention(seed: int, shape) -> np.ndarray:
    """A scale attention S [B,Nq,M,L,K] for the fused prologue: U(0, 2), a
    predicted per-point factor (the pages give no distribution)."""
    return _rng(seed).uniform(0.0, 2.0, shape).astype(np.float32)


def fused_case(seed: int, B: int, shapes, Nq: int, M: int, D: int, K: int,
               ref_low: float = 0.0, ref_high: float = 1.0, sigma_px: float = 2.0,
               logit_scale: float = 1.0, bf16: bool = False,
               with_scale: bool = False) -> FusedWorkload:
    """Small random case for the fused prologue: references uniform in
    [ref_low, ref_high) per level, offsets N(0, sigma_px) pixels, logits
    N(0, logit_scale); with_scale adds a scale attention (seed + 6)."""
    ss, st = level_table(shapes)
    Nv = int(ss.prod(axis=1).sum()) if len(shapes) else 0
    L = len(shapes)
    r = _rng(seed)
    vals = r.standard_normal((B, Nv, M, D)).astype(np.float32)
    ref = r.uniform(ref_low, ref_high, (B, Nq, L, 2)).astype(np.float32)
    off = (r.standard_normal((B, Nq, M, L, K, 2)) * sigma_px).astype(np.float32)
    logits = (r.standard_normal((B, Nq, M, L * K)) * logit_scale).astype(np.float32)
    g = r.standard_normal((B, Nq, M * D)).astype(np.float32)
    S = scale_attention(seed + 6, (B, Nq, M, L, K)) if with_scale else None
    name = f"fused_random(seed={seed})"
    if bf16:
        bits = bf16_bits(vals)
        return FusedWorkload(name, bf16_to_f32(bits).reshape(vals.shape), ss, st, ref, off,
                             logits, g, value_bf16=bits.reshape(vals.shape), attn_scale=S)
    return FusedWorkload(name, vals, ss, st, ref, off, logits, g, attn_scale=S)


def make_fused(config: int | str = "encoder_bwd", batch: Optional[int] = None,
               with_scale: bool = False) -> FusedWorkload:
    """The encoder-shape configurations in the fused prologue's input form:
    every flattened pixel is a query whose reference point is its own pixel
    centre on every level, offsets N(0, sigma) pixels of each level and
    logits N(0, 1) (seeds 1000*config + 2 and + 3, as in make()); with_scale
    adds a scale attention (seed 1000*config + 6)."""
    idx = CONFIG_NAMES.index(config) if isinstance(config, str) else int(config)
    if idx not in (1, 3, 4):
        raise ValueError("fused inputs are defined for the encoder-shape configurations")
    base = 1000 * idx
    shapes = DETR_LEVELS
    ss, st = level_table(shapes)
    Nv = int(ss.prod(axis=1).sum())
    L = len(shapes)
    M, D = 8, 32
    B, K, sigma = (2, 4, 2.0) if idx in (1, 3) else (4, 8, 3.0)
    if batch is not None:
        B = int(batch)
    Nq = Nv
    vals = _rng(base + 0).standard_normal((B, Nv, M, D)).astype(np.float32)
    ref = np.broadcast_to(_encoder_refs(shapes)[None, :, None, :], (B, Nq, L, 2))
    ref = np.ascontiguousarray(ref, dtype=np.float32)
    off = (_rng(base + 2).standard_normal((B, Nq, M, L, K, 2)) * sigma).astype(np.float32)
    logits = _rng(base + 3).standard_normal((B, Nq, M, L * K)).astype(np.float32)
    g = _rng(base + 4).standard_normal((B, Nq, M * D)).astype(np.float32)
    S = scale_attention(base + 6, (B, Nq, M, L, K)) if with_scale else None
    name = CONFIG_NAMES[idx] + "_fused"
    if idx == 4:
        bits = bf16_bits(vals)
        return FusedWorkload(name, bf16_to_f32(bits).reshape(vals.shape), ss, st, ref, off,
                             logits, g, value_bf16=bits.reshape(vals.shape), attn_scale=S)
    return FusedWorkload(name, vals, ss, st, ref, off, logits, g, attn_scale=S)


# ---------------------------------------------------------------------------
# 3-D (trilinear) variant: voxel pyramids
# ---------------------------------------------------------------------------
VOXEL_LEVELS: Tuple[Tuple[int, int, int], ...] = ((4, 128, 128), (2, 64, 64), (1, 32, 32))


def volume_table(shapes: Sequence[Tuple[int, int, int]]):
    """(shapes int64 [L,3] rows (Z,H,W), level_start_index int64 [L])."""
    ss = np.asarray(shapes, dtype=np.int64).reshape(-1, 3)
    sizes = ss[:, 0] * ss[:, 1] * ss[:, 2]
    start = np.zeros(len(ss), dtype=np.int64)
    if len(ss) > 1:
        start[1:] = np.cumsum(sizes)[:-1]
    return ss, start


def volume_case(seed: int, B: int, shapes, Nq: int, M: int, D: int, K: int,
                loc_low: float = -0.1, loc_high: float = 1.1, bf16: bool = False) -> Workload:
    """Small random 3-D case: locations [B,Nq,M,L,K,3] iid uniform per coordinate."""
    ss, st = volume_table(shapes)
    Nv = int(ss.prod(axis=1).sum()) if len(shapes) else 0
    L = len(shapes)
    r = _rng(seed)
    vals = r.standard_normal((B, Nv, M, D)).astype(np.float32)
    loc = r.uniform(loc_low, loc_high, (B, Nq, M, L, K, 3)).astype(np.float32)
    logits = r.standard_normal((B, Nq, M, L * K))
    w = softmax_lastaxis(logits).reshape(B, Nq, M, L, K).astype(np.float32)
    g = r.standard_normal((B, Nq, M * D)).astype(np.float32)
    name = f"volume_random(seed={seed})"
    if bf16:
        bits = bf16_bits(vals)
        return Workload(name, bf16_to_f32(bits).reshape(vals.shape), ss, st, loc, w, g,
                        value_bf16=bits.reshape(vals.shape), value_unrounded=vals)
    return Workload(name, vals, ss, st, loc, w, g)


def make_volume(batch: int = 1) -> Workload:
    """The voxel workload of the 3-D variant: a three-level voxel pyramid
    (Z,H,W) = 4x128x128, 2x64x64, 1x32x32 (74,752 voxels), one query per
    cell of the 128x128 bird's-eye grid (Nq = 16,384) whose reference is the
    cell centre at a height drawn U(0.1, 0.9), offsets N(0, 2 voxels of each
    level) on every axis, M=8, D=32, K=4, softmax weights, fp32.  Seeds
    9000 + tensor id."""
    shapes = VOXEL_LEVELS
    ss, st = volume_table(shapes)
    Nv = int(ss.prod(axis=1).sum())
    L, M, D, K = len(shapes), 8, 32, 4
    Hq = Wq = 128
    Nq = Hq * Wq
    B = int(batch)
    base = 9000
    vals = _rng(base + 0).standard_normal((B, Nv, M, D)).astype(np.float32)
    ys, xs = np.meshgrid((np.arange(Hq) + 0.5) / Hq, (np.arange(Wq) + 0.5) / Wq, indexing="ij")
    zs = _rng(base + 1).uniform(0.1, 0.9, (B, Nq))
    ref = np.stack([np.broadcast_to(xs.ravel(), (B, Nq)), np.broadcast_to(ys.ravel(), (B, Nq)),
                    zs], axis=-1)                                             # [B, Nq, 3]
    off = _rng(base + 2).standard_normal((B, Nq, M, L, K, 3)) * 2.0
    whz = np.array([[w, h, z] for (z, h, w) in shapes], dtype=np.float64)   # [L, 3] (W,H,Z)
    loc = (ref[:, :, None, None, None, :] + off / whz[None, None, None, :, None, :])
    w = _weights(base + 3, B, Nq, M, L, K)
    g = _rng(base + 4).standard_normal((B, Nq, M * D)).astype(np.float32)
    return Workload("volume", vals, ss, st, loc.astype(np.float32), w, g)


# ---------------------------------------------------------------------------
# DAT sampled-key attention
# ---------------------------------------------------------------------------
@dataclasses.dataclass
class DatWorkload:
    """Inputs of DAT's deformable sampling and of its attention."""
    name: str
    x: np.ndarray                     # [B, H*W, G, Dg] float32 features, channel-last
    hw: Tuple[int, int]               # (H, W)
    pos: np.ndarray                   # [B, Ns, G, 2] float32 normalized sampling positions (u, v)
    q: np.ndarray                     # [B, N, Hh, d] float32
    k: np.ndarray                     # [B, Ns, Hh, d] float32
    v: np.ndarray                     # [B, Ns, Hh, d] float32
    bias: Optional[np.ndarray]        # [B, Hh, N, Ns] float32 or None
    grad_out: np.ndarray              # [B, N, Hh, d] float32
    grad_sampled: np.ndarray          # [B, Ns, G*Dg] float32

    @property
    def dims(self):
        B, N, Hh, d = self.q.shape
        Ns = self.k.shape[1]
        _, _, G, Dg = self.x.shape
        return dict(B=B, N=N, Ns=Ns, Hh=Hh, d=d, G=G, Dg=Dg, H=self.hw[0], W=self.hw[1])


DAT_CONFIGS = {
    # DAT-T stage 3 at 224x224 (14x14 tokens, 384 channels, 12 heads of 32,
    # 6 offset groups, reference grid 7x7 = 49 sampled keys), batch 64
    "dat_cls": dict(B=64, H=14, W=14, C=384, heads=12, G=6, r=2),
    # the same stage at 1024x1024 input for detection (64x64 tokens,
    # reference grid 16x16 = 256 keys), batch 2
    "dat_det": dict(B=2, H=64, W=64, C=384, heads=12, G=6, r=4),
}


def dat_case(seed: int, B: int, H: int, W: int, C: int, heads: int, G: int, Hk: int, Wk: int,
             with_bias: bool = True, offset_cells: float = 0.5, name: str = "") -> DatWorkload:
    """Features N(0,1); sampling positions = reference-grid cell centres plus
    N(0, offset_cells) cells; q, k, v N(0,1) (the projections are outside
    this path); bias N(0, 0.5) when asked for; upstream gradients N(0,1)."""
    r = _rng(seed)
    Dg, d = C // G, C // heads
    N, Ns = H * W, Hk * Wk
    x = r.standard_normal((B, N, G, Dg)).astype(np.float32)
    gy, gx = np.meshgrid((np.arange(Hk) + 0.5) / Hk, (np.arange(Wk) + 0.5) / Wk, indexing="ij")
    ref = np.stack([gx.ravel(), gy.ravel()], axis=-1)                      # [Ns, 2] (u, v)
    off = r.standard_normal((B, Ns, G, 2)) * offset_cells / np.array([Wk, Hk])
    pos = (ref[None, :, None, :] + off).astype(np.float32)
    q = r.standard_normal((B, N, heads, d)).astype(np.float32)
    k = r.standard_normal((B, Ns, heads, d)).astype(np.float32)
    v = r.standard_normal((B, Ns, heads, d)).astype(np.float32)
    bias = (r.standard_normal((B, heads, N, Ns)) * 0.5).astype(np.float32) if with_bias else None
    g = r.standard_normal((B, N, heads, d)).astype(np.float32)
    gs = r.standard_normal((B, Ns, C)).astype(np.float32)
    return DatWorkload(name or f"dat(seed={seed})", x, (H, W), pos, q, k, v, bias, g, gs)


def make_dat(name: str = "dat_det", with_bias: bool = False) -> DatWorkload:
    """One of DAT_CONFIGS (seed 8000 / 8100)."""
    c = DAT_CONFIGS[name]
    seed = 8000 if name == "dat_cls" else 8100
    return dat_case(seed, c["B"], c["H"], c["W"], c["C"], c["heads"], c["G"], c["H"] // c["r"],
                    c["W"] // c["r"], with_bias=with_bias, name=name)
