"""Pins for the fused-prologue oracle (oracle/fused.py).

Each ``pin_*`` takes the module under test (``oracle.fused`` or a copy with a
planted mistake) and raises AssertionError when it disagrees with what the
pages or the mathematics fix:

  pin_fused_autograd       torch CPU fp64 autograd through the module's own
                           steps (reference + offset / (W_l, H_l), softmax,
                           per-level grid_sample), forward and every gradient,
                           for both softmax groupings and both pixel conventions
  pin_fused_initial_state  zero offsets and equal logits sample every level at
                           the reference point with uniform weights (first
                           page, section 3.2: the zero initialisation of the
                           offset and weight branches), a closed form
  pin_fused_logit_shift    a constant added to the logits of one softmax group
                           changes nothing; added per level it changes the
                           global-softmax output but not the per-level one
  pin_fused_translation    moving a reference point by n pixels of its level
                           and the offsets by -n pixels keeps every location
  pin_fused_softmax_grad   the logit gradients of one softmax group sum to zero
  pin_fused_shift_gradient the same translation symmetry, differentiated: the
                           reference gradient equals the offset gradients
                           times (W_l, H_l), summed over heads and points
  pin_fused_finite_differences central differences along random directions of
                           the offsets, the references and the logits, with
                           every location kept inside its bilinear cell
  pin_fused_scale_autograd the scale attention S of the "Deformable DETR"
                           tutorial (section 3.3, weight S * A): torch CPU fp64
                           autograd through the module's steps with the extra
                           factor, forward and every gradient including S's
  pin_fused_scale_identity S = 1 gives exactly the unscaled results
  pin_fused_scale_linear   the output is linear in S (superposition, S = 0
                           samples nothing) and central differences along S,
                           exact for a linear map, equal <grad_scale, dS>
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads
from oracle_pins import grid_sample_core, max_rel

SHAPES = ((6, 7), (3, 5))


def _case(seed=11, K=3, **kw):
    return workloads.fused_case(seed, 2, SHAPES, 5, 2, 4, K, **kw)


def _torch_fused(w, per_level, align, scale=None):
    """fp64 autograd of the module's forward steps written with torch ops
    (with scale: the weights are S * softmax; S's gradient is returned last)."""
    B, Nq, M, L, K, _ = w.sampling_offsets.shape
    v = torch.tensor(w.value, dtype=torch.float64, requires_grad=True)
    ref = torch.tensor(w.reference_points, dtype=torch.float64, requires_grad=True)
    off = torch.tensor(w.sampling_offsets, dtype=torch.float64, requires_grad=True)
    z = torch.tensor(w.attn_logits, dtype=torch.float64, requires_grad=True)
    wh = torch.tensor([[W, H] for H, W in w.spatial_shapes.tolist()], dtype=torch.float64)
    loc = ref[:, :, None, :, None, :] + off / wh[None, None, None, :, None, :]
    groups = z.view(B, Nq, M, L, K) if per_level else z.view(B, Nq, M, 1, L * K)
    A = torch.softmax(groups, dim=-1).reshape(B, Nq, M, L, K)
    S = None
    if scale is not None:
        S = torch.tensor(scale, dtype=torch.float64, requires_grad=True)
        A = S * A
    out = grid_sample_core(v, w.spatial_shapes, w.level_start_index, loc, A, align)
    out.backward(torch.tensor(w.grad_out, dtype=torch.float64).reshape(out.shape))
    res = (out.detach().numpy(), v.grad.numpy(), off.grad.numpy(), z.grad.numpy(),
           ref.grad.numpy())
    return res if S is None else res + (S.grad.numpy(),)


def _args(w):
    return (w.value, w.spatial_shapes, w.level_start_index, w.reference_points,
            w.sampling_offsets, w.attn_logits)


def pin_fused_autograd(impl):
    for per_level in (False, True):
        for align in (False, True):
            w = _case(seed=21 + 2 * per_level + align, ref_low=-0.05, ref_high=1.05)
            mode = oracle.DOUBLE | (oracle.ALIGN if align else 0)
            t_out, t_gv, t_goff, t_gz, t_gref = _torch_fused(w, per_level, align)
            out = impl.forward(*_args(w), per_level=per_level, mode=mode)
            gv, goff, gz, gref = impl.backward(*_args(w), w.grad_out, per_level=per_level,
                                               mode=mode)
            tag = f"per_level={per_level} align={align}"
            # the oracle rounds locations to fp32 (1 ulp ~ 6e-8): tolerances allow for it
            assert max_rel(out, t_out) < 1e-6, tag
            assert max_rel(gv, t_gv) < 1e-6, tag
            assert goff.shape == t_goff.shape and max_rel(goff, t_goff) < 1e-5, tag
            assert gz.shape == t_gz.shape and max_rel(gz, t_gz) < 1e-5, tag
            assert gref.shape == t_gref.shape and max_rel(gref, t_gref) < 1e-5, tag


def pin_fused_initial_state(impl):
    # reference at the centre of pixel (px_l, py_l) of every level, no offset,
    # equal logits: each level's K points all sample that pixel's value
    w = _case(seed=31)
    B, Nq, M, L, K, _ = w.sampling_offsets.shape
    r = np.random.Generator(np.random.PCG64(5))
    ref = np.zeros((B, Nq, L, 2), np.float32)
    expect_sum = np.zeros((B, Nq, M, w.value.shape[-1]))
    for l, (H, W) in enumerate(w.spatial_shapes.tolist()):
        px = r.integers(0, W, (B, Nq))
        py = r.integers(0, H, (B, Nq))
        ref[:, :, l, 0] = (px + 0.5) / W
        ref[:, :, l, 1] = (py + 0.5) / H
        pix = w.level_start_index[l] + py * W + px
        expect_sum += w.value[np.arange(B)[:, None], pix]          # [B, Nq, M, D]
    off = np.zeros_like(w.sampling_offsets)
    z = np.full_like(w.attn_logits, 0.75)
    args = (w.value, w.spatial_shapes, w.level_start_index, ref, off, z)
    glob = impl.forward(*args, per_level=False, mode=oracle.DOUBLE)
    perl = impl.forward(*args, per_level=True, mode=oracle.DOUBLE)
    # global softmax: weight 1/(L*K) on each point -> mean over levels;
    # per level: 1/K within each level -> sum over levels (the weights and the
    # pixel-centre references are rounded to fp32: ~1e-7)
    assert max_rel(glob, (expect_sum / L).reshape(glob.shape)) < 1e-6
    assert max_rel(perl, expect_sum.reshape(perl.shape)) < 1e-6


def pin_fused_logit_shift(impl):
    w = _case(seed=41, K=2)
    B, Nq, M, L, K, _ = w.sampling_offsets.shape
    r = np.random.Generator(np.random.PCG64(6))
    per_item = r.integers(-4, 5, (B, Nq, M, 1)).astype(np.float32)
    per_lvl = np.repeat(r.integers(-4, 5, (B, Nq, M, L)), K, axis=-1).astype(np.float32)
    # logits on a 2^-10 grid, so that adding small integers is exact in fp32
    z = (np.round(w.attn_logits * 1024.0) / 1024.0).astype(np.float32)
    base = (w.value, w.spatial_shapes, w.level_start_index, w.reference_points,
            w.sampling_offsets)
    for per_level in (False, True):
        ref_out = impl.forward(*base, z, per_level=per_level)
        shifted = impl.forward(*base, z + per_item, per_level=per_level)
        assert max_rel(shifted, ref_out) < 1e-12, f"per-item shift, per_level={per_level}"
    g0 = impl.forward(*base, z, per_level=False)
    g1 = impl.forward(*base, z + per_lvl, per_level=False)
    p0 = impl.forward(*base, z, per_level=True)
    p1 = impl.forward(*base, z + per_lvl, per_level=True)
    assert max_rel(p1, p0) < 1e-12, "per-level shift must not change per-level softmax"
    assert max_rel(g1, g0) > 1e-3, "per-level shift must change the global softmax"


def pin_fused_translation(impl):
    w = _case(seed=51, ref_low=0.2, ref_high=0.8)
    L = w.spatial_shapes.shape[0]
    n = np.array([[2, -1], [-1, 1]], dtype=np.float64)[:L]       # pixels (x, y) per level
    wh = np.array([[W, H] for H, W in w.spatial_shapes.tolist()], dtype=np.float64)
    ref2 = (w.reference_points + (n / wh)[None, None]).astype(np.float32)
    off2 = (w.sampling_offsets - n[None, None, None, :, None, :]).astype(np.float32)
    for per_level in (False, True):
        a = impl.forward(*_args(w), per_level=per_level)
        b = impl.forward(w.value, w.spatial_shapes, w.level_start_index, ref2, off2,
                         w.attn_logits, per_level=per_level)
        assert max_rel(b, a) < 1e-5, f"translation, per_level={per_level}"


def pin_fused_softmax_grad(impl):
    w = _case(seed=61, K=3)
    B, Nq, M, L, K, _ = w.sampling_offsets.shape
    for per_level in (False, True):
        _, _, gz, _ = impl.backward(*_args(w), w.grad_out, per_level=per_level)
        assert gz.shape == (B, Nq, M, L * K)
        groups = gz.reshape(B, Nq, M, L, K) if per_level else gz.reshape(B, Nq, M, 1, L * K)
        scale = float(np.max(np.abs(gz)))
        assert scale > 0
        assert float(np.max(np.abs(groups.sum(-1)))) < 1e-12 * scale * L * K, \
            f"group sums, per_level={per_level}"


def pin_fused_shift_gradient(impl):
    # out(ref + t*d/(W,H), off - t*d) is constant in t for any pixel shift d[b,q,l],
    # so sum grad_ref * d/(W,H) = sum grad_off * d
    w = _case(seed=71, ref_low=0.1, ref_high=0.9)
    B, Nq, M, L, K, _ = w.sampling_offsets.shape
    wh = np.array([[W, H] for H, W in w.spatial_shapes.tolist()], dtype=np.float64)
    d = np.random.Generator(np.random.PCG64(7)).standard_normal((B, Nq, L, 2))
    for per_level in (False, True):
        _, goff, _, gref = impl.backward(*_args(w), w.grad_out, per_level=per_level)
        assert gref.shape == (B, Nq, L, 2) and goff.shape == (B, Nq, M, L, K, 2)
        lhs = float(np.sum(gref * d / wh[None, None]))
        rhs = float(np.sum(goff * d[:, :, None, :, None, :]))
        assert abs(lhs - rhs) <= 1e-9 * (abs(lhs) + abs(rhs)) + 1e-12, (lhs, rhs)
        assert abs(lhs) > 1e-3


def _cell_interior_case(seed):
    # locations whose pixel coordinates sit in [0.25, 0.75] of a cell, so that
    # a perturbation of 1e-2 pixels never changes the bilinear cell
    w = _case(seed=seed)
    B, Nq, M, L, K, _ = w.sampling_offsets.shape
    r = np.random.Generator(np.random.PCG64(seed + 1))
    off = np.empty_like(w.sampling_offsets)
    for l, (H, W) in enumerate(w.spatial_shapes.tolist()):
        for a, n in ((0, W), (1, H)):
            cell = r.integers(-1, n, (B, Nq, M, K))
            x = cell + r.uniform(0.25, 0.75, (B, Nq, M, K))   # target pixel coordinate
            u = (x + 0.5) / n                                  # its normalized location
            ref = w.reference_points[:, :, l, a].astype(np.float64)[:, :, None, None]
            off[:, :, :, l, :, a] = (u - ref) * n
    w.sampling_offsets = off.astype(np.float32)
    return w


def pin_fused_finite_differences(impl):
    w = _cell_interior_case(81)
    r = np.random.Generator(np.random.PCG64(8))
    g = w.grad_out.astype(np.float64)
    for per_level in (False, True):
        _, goff, gz, gref = impl.backward(*_args(w), w.grad_out, per_level=per_level,
                                          mode=oracle.DOUBLE)

        def f(ref, off, z):
            out = impl.forward(w.value, w.spatial_shapes, w.level_start_index, ref, off, z,
                               per_level=per_level, mode=oracle.DOUBLE)
            return float(np.sum(out.reshape(g.shape) * g))

        wh = np.array([[W, H] for H, W in w.spatial_shapes.tolist()], dtype=np.float64)
        # directions: offsets in pixels, references in pixels of each level, logits
        d_off = r.standard_normal(w.sampling_offsets.shape)
        d_ref = r.standard_normal(w.reference_points.shape) / wh[None, None]
        d_z = r.standard_normal(w.attn_logits.shape)
        for name, grad, dirn, h in (("offsets", goff, d_off, 1e-2), ("ref", gref, d_ref, 1e-2),
                                    ("logits", gz, d_z, 1e-3)):
            args = [w.reference_points.astype(np.float64), w.sampling_offsets.astype(np.float64),
                    w.attn_logits.astype(np.float64)]
            k = {"ref": 0, "offsets": 1, "logits": 2}[name]
            plus = list(args)
            minus = list(args)
            plus[k] = args[k] + h * dirn
            minus[k] = args[k] - h * dirn
            fd = (f(*[a.astype(np.float32) for a in plus]) -
                  f(*[a.astype(np.float32) for a in minus])) / (2 * h)
            an = float(np.sum(grad * dirn))
            assert abs(fd - an) <= 2e-3 * abs(an) + 1e-6, (name, per_level, fd, an)


def pin_fused_scale_autograd(impl):
    for per_level, align in ((False, False), (True, False), (False, True)):
        w = _case(seed=91 + 2 * per_level + align, ref_low=-0.05, ref_high=1.05,
                  with_scale=True)
        S = w.attn_scale
        mode = oracle.DOUBLE | (oracle.ALIGN if align else 0)
        t_out, t_gv, t_goff, t_gz, t_gref, t_gs = _torch_fused(w, per_level, align, S)
        out = impl.forward(*_args(w), per_level=per_level, mode=mode, scale=S)
        res = impl.backward(*_args(w), w.grad_out, per_level=per_level, mode=mode, scale=S)
        tag = f"scale per_level={per_level} align={align}"
        assert len(res) == 5, tag
        gv, goff, gz, gref, gs = res
        # the oracle rounds S * A and the locations to fp32: tolerances allow for it
        assert max_rel(out, t_out) < 1e-6, tag
        assert max_rel(gv, t_gv) < 1e-6, tag
        assert goff.shape == t_goff.shape and max_rel(goff, t_goff) < 1e-5, tag
        assert gz.shape == t_gz.shape and max_rel(gz, t_gz) < 1e-5, tag
        assert gref.shape == t_gref.shape and max_rel(gref, t_gref) < 1e-5, tag
        assert gs.shape == t_gs.shape and max_rel(gs, t_gs) < 1e-5, tag


def pin_fused_scale_identity(impl):
    w = _case(seed=101)
    ones = np.ones(w.sampling_offsets.shape[:-1], np.float32)
    for per_level in (False, True):
        a = impl.forward(*_args(w), per_level=per_level)
        b = impl.forward(*_args(w), per_level=per_level, scale=ones)
        assert np.array_equal(a, b), f"S = 1 forward, per_level={per_level}"
        ga = impl.backward(*_args(w), w.grad_out, per_level=per_level)
        gb = impl.backward(*_args(w), w.grad_out, per_level=per_level, scale=ones)
        for x, y in zip(ga, gb[:4]):
            assert np.array_equal(x, y), f"S = 1 backward, per_level={per_level}"


def pin_fused_scale_linear(impl):
    w = _case(seed=111)
    shp = w.sampling_offsets.shape[:-1]
    r = np.random.Generator(np.random.PCG64(9))
    # S on a 2^-8 grid, so that s1 + s2 is exact in fp32
    s1 = (np.round(r.uniform(-1, 1, shp) * 256) / 256).astype(np.float32)
    s2 = (np.round(r.uniform(-1, 1, shp) * 256) / 256).astype(np.float32)
    g = w.grad_out.astype(np.float64)
    for per_level in (False, True):
        f = lambda S: impl.forward(*_args(w), per_level=per_level, mode=oracle.DOUBLE, scale=S)
        o1, o2, o12 = f(s1), f(s2), f((s1 + s2).astype(np.float32))
        assert max_rel(o12, o1 + o2) < 1e-6, f"superposition, per_level={per_level}"
        assert np.all(f(np.zeros(shp, np.float32)) == 0.0), "S = 0 samples nothing"
        # central difference along dS: exact for a map linear in S
        gs = impl.backward(*_args(w), w.grad_out, per_level=per_level, mode=oracle.DOUBLE,
                           scale=s1)[4]
        dS = r.standard_normal(shp)
        h = 0.25
        fp = float(np.sum(f((s1 + h * dS).astype(np.float32)).reshape(g.shape) * g))
        fm = float(np.sum(f((s1 - h * dS).astype(np.float32)).reshape(g.shape) * g))
        fd = (fp - fm) / (2 * h)
        an = float(np.sum(gs * dS))
        assert abs(fd - an) <= 1e-5 * abs(an) + 1e-9, (per_level, fd, an)


ALL_FUSED_PINS = [pin_fused_autograd, pin_fused_initial_state, pin_fused_logit_shift,
                  pin_fused_translation, pin_fused_softmax_grad, pin_fused_shift_gradient,
                  pin_fused_finite_differences, pin_fused_scale_autograd,
                  pin_fused_scale_identity, pin_fused_scale_linear]
