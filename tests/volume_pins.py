"""Pins for the 3-D (trilinear) oracle (oracle/msda3d_oracle.c).

Each ``pin_*`` takes an ``oracle.volume.VolumeLib`` and raises AssertionError
when it disagrees with what the pages or the mathematics fix:

  pin_volume_grid_sample    the whole core equals a per-level torch CPU
                            grid_sample on 5-D input (its 'bilinear' mode is
                            trilinear there; zeros padding) in fp64, forward
                            and autograd backward, for align_corners False and
                            True
  pin_volume_linear_field   trilinear interpolation reproduces a field that is
                            affine in (x, y, z) exactly inside the volume
  pin_volume_voxel_centres  sampling at a voxel centre returns the stored row
  pin_volume_flat_levels    one-voxel-thick levels sampled at mid-height are
                            the 2-D core (first page, section 5.3: the same
                            method with one more coordinate)
  pin_volume_finite_differences  central differences of the fp64 forward
  pin_volume_out_of_volume  points beyond the half-voxel border contribute zero
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

import oracle
import workloads
from oracle_pins import max_rel

SHAPES = ((3, 5, 6), (2, 3, 4))


def grid_sample_volume(value, shapes, start, loc, attn, align_corners=False):
    """Torch CPU composition over levels of 5-D grid_sample; keeps autograd."""
    B, Nv, M, D = value.shape
    _, Nq, _, L, K, _ = loc.shape
    out = torch.zeros(B * M, D, Nq, dtype=value.dtype)
    for l in range(L):
        Z, H, W = (int(v) for v in shapes[l])
        s = int(start[l])
        v_l = value[:, s:s + Z * H * W].reshape(B, Z, H, W, M, D).permute(0, 4, 5, 1, 2, 3)
        v_l = v_l.reshape(B * M, D, Z, H, W)
        grid = (2.0 * loc[:, :, :, l] - 1.0).permute(0, 2, 1, 3, 4).reshape(B * M, 1, Nq, K, 3)
        smp = F.grid_sample(v_l, grid, mode="bilinear", padding_mode="zeros",
                            align_corners=align_corners)       # [B*M, D, 1, Nq, K]
        a = attn[:, :, :, l].permute(0, 2, 1, 3).reshape(B * M, 1, Nq, K)
        out = out + (smp[:, :, 0] * a).sum(-1)
    return out.reshape(B, M, D, Nq).permute(0, 3, 1, 2).reshape(B, Nq, M * D)


def _run(orc, w, mode=oracle.SPEC, **over):
    a = dict(value=w.value, shapes=w.spatial_shapes, starts=w.level_start_index,
             loc=w.sampling_loc, attn=w.attn_weight)
    a.update(over)
    return a


def pin_volume_grid_sample(orc):
    for align in (False, True):
        w = workloads.volume_case(31 + align, 2, SHAPES, 7, 2, 4, 3, loc_low=-0.15,
                                  loc_high=1.15)
        v = torch.tensor(w.value, dtype=torch.float64, requires_grad=True)
        lc = torch.tensor(w.sampling_loc, dtype=torch.float64, requires_grad=True)
        at = torch.tensor(w.attn_weight, dtype=torch.float64, requires_grad=True)
        out = grid_sample_volume(v, w.spatial_shapes, w.level_start_index, lc, at, align)
        out.backward(torch.tensor(w.grad_out, dtype=torch.float64).reshape(out.shape))
        mode = oracle.DOUBLE | (oracle.ALIGN if align else 0)
        args = (w.value, w.spatial_shapes, w.level_start_index, w.sampling_loc, w.attn_weight)
        o = orc.forward(*args, mode=mode)
        gv, gl, ga = orc.backward(*args, w.grad_out, mode=mode)
        tag = f"align={align}"
        assert max_rel(o, out.detach().numpy()) < 1e-12, tag
        assert max_rel(gv, v.grad.numpy()) < 1e-12, tag
        assert max_rel(gl, lc.grad.numpy()) < 1e-10, tag
        assert max_rel(ga, at.grad.numpy()) < 1e-12, tag


def pin_volume_linear_field(orc):
    # value[voxel (x, y, z), channel d] = c0[d] + cx[d]*x + cy[d]*y + cz[d]*z:
    # trilinear interpolation is exact for it inside [0, W-1] x [0, H-1] x [0, Z-1]
    shapes = ((4, 6, 7),)
    ss, st = workloads.volume_table(shapes)
    Z, H, W = shapes[0]
    M, D, K, Nq = 1, 4, 5, 6
    r = np.random.Generator(np.random.PCG64(17))
    coef = r.integers(-3, 4, (4, D)).astype(np.float64)
    zz, yy, xx = np.meshgrid(np.arange(Z), np.arange(H), np.arange(W), indexing="ij")
    field = (coef[0] + coef[1] * xx.reshape(-1, 1) + coef[2] * yy.reshape(-1, 1) +
             coef[3] * zz.reshape(-1, 1))
    value = field.reshape(1, Z * H * W, 1, D).astype(np.float32)
    # voxel coordinates kept off the upper faces, where fp32 rounding of the
    # location could put a sliver of weight on a neighbour outside
    p = np.stack([r.uniform(0.01, W - 1.01, (1, Nq, M, 1, K)),
                  r.uniform(0.01, H - 1.01, (1, Nq, M, 1, K)),
                  r.uniform(0.01, Z - 1.01, (1, Nq, M, 1, K))], axis=-1)
    loc = ((p + 0.5) / np.array([W, H, Z])).astype(np.float32)
    onehot = np.zeros((1, Nq, M, 1, K), np.float32)
    onehot[..., 2] = 1.0
    out = orc.forward(value, ss, st, loc, onehot, mode=oracle.DOUBLE)
    pt = (loc[..., 2, :].astype(np.float64) * np.array([W, H, Z]) - 0.5)[0, :, 0, 0]
    expect = coef[0] + pt[:, 0:1] * coef[1] + pt[:, 1:2] * coef[2] + pt[:, 2:3] * coef[3]
    assert max_rel(out.reshape(Nq, D), expect) < 1e-12


def pin_volume_voxel_centres(orc):
    w = workloads.volume_case(41, 1, ((4, 8, 16), (2, 4, 8)), 9, 2, 4, 2)
    B, Nq, M, L, K, _ = w.sampling_loc.shape
    r = np.random.Generator(np.random.PCG64(9))
    loc = np.zeros_like(w.sampling_loc)
    expect = np.zeros((B, Nq, M, w.value.shape[-1]))
    attn = np.zeros_like(w.attn_weight)
    for l, (Z, H, W) in enumerate(w.spatial_shapes.tolist()):
        for q in range(Nq):
            for m in range(M):
                x, y, z = r.integers(0, W), r.integers(0, H), r.integers(0, Z)
                loc[0, q, m, l, 0] = [(x + 0.5) / W, (y + 0.5) / H, (z + 0.5) / Z]
                loc[0, q, m, l, 1] = [-5.0, 0.5, 0.5]                  # outside: no weight
                attn[0, q, m, l, 0] = 1.0
                vox = w.level_start_index[l] + (z * H + y) * W + x
                expect[0, q, m] += w.value[0, vox, m]
    out = orc.forward(w.value, w.spatial_shapes, w.level_start_index, loc, attn)
    assert np.array_equal(out.reshape(expect.shape), expect)


def pin_volume_flat_levels(orc):
    shapes2 = ((5, 7), (3, 4))
    w2 = workloads.random_case(51, 2, shapes2, 6, 2, 4, 3)
    ss3 = np.array([[1, h, wd] for h, wd in shapes2], dtype=np.int64)
    loc3 = np.concatenate([w2.sampling_loc, np.full(w2.sampling_loc.shape[:-1] + (1,), 0.5,
                                                    np.float32)], axis=-1)
    args2 = (w2.value, w2.spatial_shapes, w2.level_start_index, w2.sampling_loc, w2.attn_weight)
    args3 = (w2.value, ss3, w2.level_start_index, loc3, w2.attn_weight)
    for mode in (oracle.SPEC, oracle.DOUBLE):
        assert max_rel(orc.forward(*args3, mode=mode), oracle.forward(*args2, mode=mode)) < 1e-14
        gv3, gl3, ga3 = orc.backward(*args3, w2.grad_out, mode=mode)
        gv2, gl2, ga2 = oracle.backward(*args2, w2.grad_out, mode=mode)
        assert max_rel(gv3, gv2) < 1e-14 and max_rel(ga3, ga2) < 1e-14
        assert max_rel(gl3[..., :2], gl2) < 1e-14


def pin_volume_finite_differences(orc):
    w = workloads.volume_case(61, 1, SHAPES, 5, 2, 4, 2, loc_low=0.05, loc_high=0.95)
    g = w.grad_out.astype(np.float64)
    args = dict(shapes=w.spatial_shapes, starts=w.level_start_index)
    gv, gl, ga = orc.backward(w.value, w.spatial_shapes, w.level_start_index, w.sampling_loc,
                              w.attn_weight, w.grad_out, mode=oracle.DOUBLE)

    def f(value, loc, attn):
        out = orc.forward(value, args["shapes"], args["starts"], loc, attn, mode=oracle.DOUBLE)
        return float(np.sum(out.reshape(g.shape) * g))

    r = np.random.Generator(np.random.PCG64(12))
    # one coordinate at a time, all points at once along a random direction;
    # within its cell a point's sample is linear in each coordinate, so the
    # difference over the fp32-rounded locations is exact up to fp64 rounding.
    # Points whose cell would change are held still.
    loc = w.sampling_loc
    for a in range(3):
        ext = w.spatial_shapes[:, 2 - a].astype(np.float64)[None, None, None, :, None]  # W, H, Z
        d = r.standard_normal(loc.shape[:-1]) * 1e-3 / ext
        lp, lm = loc.copy(), loc.copy()
        lp[..., a] = (loc[..., a] + d).astype(np.float32)
        lm[..., a] = (loc[..., a] - d).astype(np.float32)
        same = np.floor(lp[..., a] * ext - 0.5) == np.floor(lm[..., a] * ext - 0.5)
        lp[..., a] = np.where(same, lp[..., a], loc[..., a])
        lm[..., a] = np.where(same, lm[..., a], loc[..., a])
        delta = lp[..., a].astype(np.float64) - lm[..., a].astype(np.float64)
        fd = f(w.value, lp, w.attn_weight) - f(w.value, lm, w.attn_weight)
        an = float(np.sum(gl[..., a] * delta))
        assert abs(fd - an) <= 1e-8 * abs(an) + 1e-12, (a, fd, an)
        assert same.mean() > 0.9
    # the output is linear in the weights and in value: exact differences
    ap = (w.attn_weight + 0.25 * r.standard_normal(w.attn_weight.shape)).astype(np.float32)
    fd = f(w.value, w.sampling_loc, ap) - f(w.value, w.sampling_loc, w.attn_weight)
    an = float(np.sum(ga * (ap.astype(np.float64) - w.attn_weight)))
    assert abs(fd - an) <= 1e-10 * abs(an) + 1e-12
    vp = (w.value + 0.5 * r.standard_normal(w.value.shape)).astype(np.float32)
    fd = f(vp, w.sampling_loc, w.attn_weight) - f(w.value, w.sampling_loc, w.attn_weight)
    an = float(np.sum(gv * (vp.astype(np.float64) - w.value)))
    assert abs(fd - an) <= 1e-10 * abs(an) + 1e-12


def pin_volume_out_of_volume(orc):
    w = workloads.volume_case(71, 1, SHAPES, 4, 2, 4, 2)
    loc = w.sampling_loc.copy()
    # a point is outside once its voxel coordinate is below -1 or above n,
    # i.e. u < -0.5/n or u > 1 + 0.5/n; the extents here are 2..6 voxels
    for axis, u in ((0, -0.6), (1, 1.21)):
        far = loc.copy()
        far[..., axis] = u
        out = orc.forward(w.value, w.spatial_shapes, w.level_start_index, far, w.attn_weight)
        assert float(np.max(np.abs(out))) == 0.0
    z_far = loc.copy()
    z_far[..., 2] = 1.3
    out = orc.forward(w.value, w.spatial_shapes, w.level_start_index, z_far, w.attn_weight)
    gv, gl, ga = orc.backward(w.value, w.spatial_shapes, w.level_start_index, z_far,
                              w.attn_weight, w.grad_out)
    assert float(np.max(np.abs(out))) == 0.0
    assert float(np.max(np.abs(gv))) == 0.0 and float(np.max(np.abs(gl))) == 0.0
    assert float(np.max(np.abs(ga))) == 0.0


ALL_VOLUME_PINS = [pin_volume_grid_sample, pin_volume_linear_field, pin_volume_voxel_centres,
                   pin_volume_flat_levels, pin_volume_finite_differences,
                   pin_volume_out_of_volume]
