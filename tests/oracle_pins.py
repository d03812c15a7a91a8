"""Pins for the CPU oracle: checks against facts that do not come from the oracle.

Each ``pin_*`` takes an ``oracle.OracleLib`` and raises AssertionError when
the oracle disagrees with what the pages or the mathematics fix:

  pin_pixel_centres      sampling at a pixel centre returns the stored value
  pin_one_hot_grid_sample one-hot weights reproduce one bilinear sample, and the
                         whole core equals a per-level torch grid_sample
                         (bilinear, zeros, align_corners=False) on CPU, fp64,
                         forward and autograd backward
  pin_four_point_example the worked example of the engineering-notes page
  pin_zero_offsets       zero offsets reduce to a gather at the reference
  pin_finite_differences central differences of the forward (fp64 mode)
  pin_adjoint            <g, F(dv)> = <F^T g, dv> and the same for the weights
  pin_partition_of_unity a constant field is reproduced by weights summing to 1
  pin_out_of_map         points beyond the half-pixel border contribute zero
  pin_nonfinite          NaN/Inf locations contribute zero and get zero grads
  pin_linearity          the output is linear in the attention weights

The mutant test compiles copies of the oracle with one planted mistake each
and requires every copy to fail at least one pin.
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch
import torch.nn.functional as F

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def max_rel(x, r) -> float:
    x = np.asarray(x, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    den = float(np.max(np.abs(r))) if r.size else 0.0
    num = float(np.max(np.abs(x - r))) if r.size else 0.0
    if den == 0.0:
        return num
    return num / den


# ----------------------------------------------------------------------------
# torch grid_sample composition (library routine the per-level sampling reduces
# to: first page, section 3.2 -- grid = 2*loc - 1, bilinear, zero padding,
# align_corners=False, heads folded into the batch).
# ----------------------------------------------------------------------------
def grid_sample_core(value, shapes, start, loc, attn, align_corners=False):
    """Torch CPU composition; tensors in, out [B, Nq, M*D] (keeps autograd)."""
    B, Nv, M, D = value.shape
    _, Nq, _, L, K, _ = loc.shape
    out = torch.zeros(B * M, D, Nq, dtype=value.dtype)
    for l in range(L):
        H, W = int(shapes[l][0]), int(shapes[l][1])
        s = int(start[l])
        v_l = value[:, s:s + H * W].reshape(B, H, W, M, D).permute(0, 3, 4, 1, 2)
        v_l = v_l.reshape(B * M, D, H, W)
        grid = (2.0 * loc[:, :, :, l] - 1.0).permute(0, 2, 1, 3, 4).reshape(B * M, Nq, K, 2)
        smp = F.grid_sample(v_l, grid, mode="bilinear", padding_mode="zeros",
                            align_corners=align_corners)       # [B*M, D, Nq, K]
        a = attn[:, :, :, l].permute(0, 2, 1, 3).reshape(B * M, 1, Nq, K)
        out = out + (smp * a).sum(-1)
    return out.reshape(B, M, D, Nq).permute(0, 3, 1, 2).reshape(B, Nq, M * D)


def torch_reference(w: workloads.Workload, align_corners=False):
    """fp64 forward + autograd grads of the grid_sample composition."""
    v = torch.tensor(w.value, dtype=torch.float64, requires_grad=True)
    lc = torch.tensor(w.sampling_loc, dtype=torch.float64, requires_grad=True)
    a = torch.tensor(w.attn_weight, dtype=torch.float64, requires_grad=True)
    out = grid_sample_core(v, w.spatial_shapes, w.level_start_index, lc, a, align_corners)
    g = torch.tensor(w.grad_out, dtype=torch.float64).reshape(out.shape)
    out.backward(g)
    return (out.detach().numpy(), v.grad.numpy(), lc.grad.numpy(), a.grad.numpy())


def _fwd(orc, w, mode=oracle.SPEC, **over):
    args = dict(value=w.value, spatial_shapes=w.spatial_shapes,
                level_start_index=w.level_start_index, sampling_loc=w.sampling_loc,
                attn_weight=w.attn_weight)
    args.update(over)
    return orc.forward(args["value"], args["spatial_shapes"], args["level_start_index"],
                       args["sampling_loc"], args["attn_weight"], mode=mode)


def _bwd(orc, w, mode=oracle.SPEC, **over):
    args = dict(value=w.value, spatial_shapes=w.spatial_shapes,
                level_start_index=w.level_start_index, sampling_loc=w.sampling_loc,
                attn_weight=w.attn_weight, grad_out=w.grad_out)
    args.update(over)
    return orc.backward(args["value"], args["spatial_shapes"], args["level_start_index"],
                        args["sampling_loc"], args["attn_weight"], args["grad_out"],
                        mode=mode)


# ----------------------------------------------------------------------------
def pin_pixel_centres(orc):
    """A location at the centre of pixel (i, j), ((j+0.5)/W, (i+0.5)/H), maps to
    integer pixel coordinates and returns value[i, j] (first page, section 2.3:
    the neighbour at distance 0 has tent weight 1, the others 0).  Exact for
    power-of-two sizes; within 1e-6 otherwise (fp32 rounding of u*W - 0.5)."""
    for shapes, tol in ((((8, 8), (4, 4)), 0.0), (((5, 7), (3, 2), (1, 1)), 1e-6)):
        w = workloads.random_case(11, 2, shapes, 12, 3, 8, 2)
        B, Nq, M, L, K = w.attn_weight.shape
        rng = np.random.Generator(np.random.PCG64(5))
        loc = w.sampling_loc.copy()
        attn = np.zeros_like(w.attn_weight)
        expect = np.zeros((B, Nq, M, 8))
        for b in range(B):
            for q in range(Nq):
                for m in range(M):
                    l = int(rng.integers(L))
                    k = int(rng.integers(K))
                    H, W = w.spatial_shapes[l]
                    i, j = int(rng.integers(H)), int(rng.integers(W))
                    loc[b, q, m, l, k] = (np.float32((j + 0.5) / W), np.float32((i + 0.5) / H))
                    attn[b, q, m, l, k] = 1.0
                    expect[b, q, m] = w.value[b, w.level_start_index[l] + i * W + j, m]
        got = _fwd(orc, w, sampling_loc=loc, attn_weight=attn).reshape(B, Nq, M, 8)
        err = float(np.max(np.abs(got - expect)))
        assert err <= tol, f"pixel-centre sample off by {err} (shapes {shapes})"


def pin_one_hot_grid_sample(orc):
    """Forward and all three gradients equal the per-level grid_sample
    composition (torch CPU, fp64) on the tiny config and on random shapes with
    points inside, across and beyond the border; one-hot weights pick one
    bilinear sample."""
    cases = [workloads.make(0),
             workloads.random_case(21, 2, ((5, 7), (3, 4), (2, 1)), 9, 3, 4, 3),
             workloads.random_case(22, 1, ((6, 6),), 7, 1, 2, 5, -0.6, 1.6),
             workloads.random_case(23, 2, ((1, 9), (4, 1)), 5, 2, 3, 2)]
    for w in cases:
        out, gv, gl, ga = torch_reference(w)
        o = _fwd(orc, w, mode=oracle.DOUBLE)
        assert max_rel(o, out) < 1e-12, f"forward vs grid_sample on {w.name}"
        v, l_, a = _bwd(orc, w, mode=oracle.DOUBLE)
        assert max_rel(v, gv) < 1e-12, f"grad_value vs autograd on {w.name}"
        assert max_rel(l_, gl) < 1e-9, f"grad_loc vs autograd on {w.name}"
        assert max_rel(a, ga) < 1e-12, f"grad_attn vs autograd on {w.name}"
    # one-hot weights select exactly one sample of the composition
    w = cases[1]
    B, Nq, M, L, K = w.attn_weight.shape
    for (l, k) in ((0, 0), (1, 2), (2, 1)):
        onehot = np.zeros_like(w.attn_weight)
        onehot[:, :, :, l, k] = 1.0
        o = _fwd(orc, w, mode=oracle.DOUBLE, attn_weight=onehot)
        v = torch.tensor(w.value, dtype=torch.float64)
        ref = grid_sample_core(v, w.spatial_shapes, w.level_start_index,
                               torch.tensor(w.sampling_loc, dtype=torch.float64),
                               torch.tensor(onehot, dtype=torch.float64)).numpy()
        assert max_rel(o, ref) < 1e-12, f"one-hot ({l},{k}) sample"


def pin_four_point_example(orc):
    """The engineering-notes page (section 2.2) prints: reference (0.3, 0.7)
    plus offsets (+-0.1, 0), (0, +-0.1) gives (0.4,0.7), (0.2,0.7), (0.3,0.8),
    (0.3,0.6).  On a 10x10 level those are pixel midpoints of 2x2 quads, so
    each sample is the plain mean of its four neighbours."""
    ex = json.load(open(os.path.join(GOLDEN, "four_point_example.json")))
    ref = np.array(ex["reference"], dtype=np.float32)
    offs = np.array(ex["offsets"], dtype=np.float32)
    locs = ref[None, :] + offs
    assert np.max(np.abs(locs - np.array(ex["locations"], dtype=np.float32))) <= 1e-7
    H, W = ex["level_hw"]
    rng = np.random.Generator(np.random.PCG64(77))
    D = 6
    value = rng.standard_normal((1, H * W, 1, D)).astype(np.float32)
    shapes, start = workloads.level_table([(H, W)])
    img = value[0, :, 0, :].reshape(H, W, D)
    for kk, (px, py) in enumerate(ex["pixel_coords"]):
        loc = np.zeros((1, 1, 1, 1, 4, 2), np.float32)
        loc[0, 0, 0, 0, :, :] = locs
        attn = np.zeros((1, 1, 1, 1, 4), np.float32)
        attn[0, 0, 0, 0, kk] = 1.0
        got = orc.forward(value, shapes, start, loc, attn)[0, 0]
        x0, y0 = int(np.floor(px)), int(np.floor(py))
        expect = img[y0:y0 + 2, x0:x0 + 2].reshape(4, D).astype(np.float64).mean(axis=0)
        assert np.max(np.abs(got - expect)) <= 1e-6, f"point {kk}: {got} vs {expect}"
    # all four together with equal weights: mean of the four quad means
    loc = np.zeros((1, 1, 1, 1, 4, 2), np.float32)
    loc[0, 0, 0, 0] = locs
    attn = np.full((1, 1, 1, 1, 4), 0.25, np.float32)
    got = orc.forward(value, shapes, start, loc, attn)[0, 0]
    quads = [img[int(np.floor(py)):int(np.floor(py)) + 2,
                 int(np.floor(px)):int(np.floor(px)) + 2].reshape(4, D).astype(np.float64).mean(0)
             for (px, py) in ex["pixel_coords"]]
    assert np.max(np.abs(got - np.mean(quads, axis=0))) <= 1e-6


def pin_zero_offsets(orc):
    """With zero offsets every point sits on the reference; an encoder query
    at the centre of its own pixel then gathers that pixel exactly on its own
    level (first page, section 3.2: zero-initialised offsets sample at the
    reference), and other levels give the plain bilinear sample there."""
    shapes = ((6, 8), (3, 4), (2, 2))
    ss, st = workloads.level_table(shapes)
    Nv = int(ss.prod(1).sum())
    B, M, D, K, L = 2, 2, 5, 3, len(shapes)
    rng = np.random.Generator(np.random.PCG64(31))
    value = rng.standard_normal((B, Nv, M, D)).astype(np.float32)
    refs = []
    own = []
    for l, (H, W) in enumerate(shapes):
        for i in range(H):
            for j in range(W):
                refs.append(((j + 0.5) / W, (i + 0.5) / H))
                own.append(l)
    refs = np.array(refs, dtype=np.float32)
    loc = np.broadcast_to(refs[None, :, None, None, None, :], (B, Nv, M, L, K, 2)).copy()
    logits = rng.standard_normal((B, Nv, M, L * K))
    attn = workloads.softmax_lastaxis(logits).reshape(B, Nv, M, L, K).astype(np.float32)
    got = orc.forward(value, ss, st, loc, attn).reshape(B, Nv, M, D)
    # expected: own level is an exact gather, others via grid_sample
    v = torch.tensor(value, dtype=torch.float64)
    for l in range(L):
        a_l = np.zeros_like(attn)
        a_l[:, :, :, l] = attn[:, :, :, l]
        part = orc.forward(value, ss, st, loc, a_l).reshape(B, Nv, M, D)
        ref = grid_sample_core(v, ss, st, torch.tensor(loc, dtype=torch.float64),
                               torch.tensor(a_l, dtype=torch.float64)).numpy().reshape(B, Nv, M, D)
        assert max_rel(part, ref) < 1e-6, f"level {l} term"
        mask = np.array(own) == l
        gather = value[:, mask] * attn[:, mask][:, :, :, l].sum(-1, dtype=np.float64)[..., None]
        assert np.max(np.abs(part[:, mask] - gather)) <= 1e-5, f"own-level gather {l}"
    total = sum(orc.forward(value, ss, st, loc, np.where(
        np.arange(L)[None, None, None, :, None] == l, attn, 0)).reshape(B, Nv, M, D)
        for l in range(L))
    assert max_rel(got, total) < 1e-12


def pin_finite_differences(orc):
    """Central differences of the fp64 forward match the backward.  Inside a
    pixel cell the sample is linear in x and in y separately, so the central
    difference is exact up to rounding; points within 2h of a cell edge are
    skipped.  The output is linear in value and in the weights."""
    w = workloads.random_case(41, 1, ((5, 6), (3, 3)), 6, 2, 4, 2, 0.05, 0.95)
    gv, gl, ga = _bwd(orc, w, mode=oracle.DOUBLE)
    g = w.grad_out.astype(np.float64)

    def obj(**over):
        return float(np.sum(_fwd(orc, w, mode=oracle.DOUBLE, **over) * g))

    B, Nq, M, L, K = w.attn_weight.shape
    checked = 0
    rng = np.random.Generator(np.random.PCG64(3))
    for _ in range(40):
        b, q, m, l, k = (int(rng.integers(n)) for n in (B, Nq, M, L, K))
        H, W = w.spatial_shapes[l]
        for c, n in ((0, W), (1, H)):
            u = float(w.sampling_loc[b, q, m, l, k, c])
            p = u * n - 0.5
            h = 1e-3 / n
            if abs(p - np.round(p)) < 4e-3 or p < -1 or p > n:
                continue
            lp = w.sampling_loc.copy()
            lm = w.sampling_loc.copy()
            lp[b, q, m, l, k, c] = u + h
            lm[b, q, m, l, k, c] = u - h
            hh = float(lp[b, q, m, l, k, c]) - float(lm[b, q, m, l, k, c])
            fd = (obj(sampling_loc=lp) - obj(sampling_loc=lm)) / hh
            an = gl[b, q, m, l, k, c]
            assert abs(fd - an) <= 1e-4 * max(1.0, abs(an)), f"grad_loc fd {fd} vs {an}"
            checked += 1
        ap = w.attn_weight.copy()
        am = w.attn_weight.copy()
        ap[b, q, m, l, k] += np.float32(0.25)
        am[b, q, m, l, k] -= np.float32(0.25)
        hh = float(ap[b, q, m, l, k]) - float(am[b, q, m, l, k])
        fd = (obj(attn_weight=ap) - obj(attn_weight=am)) / hh
        assert abs(fd - ga[b, q, m, l, k]) <= 1e-9 * max(1.0, abs(fd)), "grad_attn fd"
    assert checked >= 20
    for _ in range(10):
        idx = tuple(int(rng.integers(n)) for n in w.value.shape)
        vp = w.value.copy()
        vm = w.value.copy()
        vp[idx] += np.float32(0.5)
        vm[idx] -= np.float32(0.5)
        fd = (obj(value=vp) - obj(value=vm)) / (float(vp[idx]) - float(vm[idx]))
        assert abs(fd - gv[idx]) <= 1e-9 * max(1.0, abs(fd)), "grad_value fd"


def pin_adjoint(orc):
    """The forward is linear in value and in the weights, so the backward must
    be its adjoint: <g, F(dv)> = <grad_value(g), dv> and likewise for A."""
    w = workloads.random_case(51, 2, ((7, 5), (4, 3), (2, 2)), 10, 3, 6, 3)
    gv, _, ga = _bwd(orc, w, mode=oracle.DOUBLE)
    g = w.grad_out.astype(np.float64)
    rng = np.random.Generator(np.random.PCG64(9))
    dv = rng.standard_normal(w.value.shape).astype(np.float32)
    lhs = float(np.sum(g * _fwd(orc, w, mode=oracle.DOUBLE, value=dv)))
    rhs = float(np.sum(gv * dv))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs)), f"value adjoint {lhs} vs {rhs}"
    da = rng.standard_normal(w.attn_weight.shape).astype(np.float32)
    lhs = float(np.sum(g * _fwd(orc, w, mode=oracle.DOUBLE, attn_weight=da)))
    rhs = float(np.sum(ga * da))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs)), f"weight adjoint {lhs} vs {rhs}"


def pin_partition_of_unity(orc):
    """Tent weights of the four neighbours sum to one, so a constant field c
    with every neighbour inside the map gives c * sum(A), and the total of
    grad_value over pixels is sum(A) * g."""
    w = workloads.random_case(61, 2, ((6, 9), (4, 4)), 8, 2, 3, 2, 0.3, 0.7)
    c = np.float32(1.75)
    const = np.full_like(w.value, c)
    o = _fwd(orc, w, value=const)
    B, Nq, M, L, K = w.attn_weight.shape
    sA = w.attn_weight.astype(np.float64).sum(axis=(3, 4))            # [B,Nq,M]
    expect = np.repeat(sA[..., None] * float(c), 3, axis=-1).reshape(B, Nq, M * 3)
    assert max_rel(o, expect) < 1e-12
    gv, _, _ = _bwd(orc, w)
    g = w.grad_out.astype(np.float64).reshape(B, Nq, M, 3)
    tot = gv.sum(axis=1)                                              # [B,M,D]
    expect = np.einsum("bqm,bqmd->bmd", sA, g)
    assert max_rel(tot, expect) < 1e-12


def pin_out_of_map(orc):
    """A point whose pixel coordinate is <= -1 or >= W (likewise H) has no
    neighbour inside the map: zero output, zero gradients (first page,
    section 2.3: out-of-map samples contribute zero)."""
    w = workloads.random_case(71, 1, ((6, 5), (3, 3)), 6, 2, 4, 3)
    loc = w.sampling_loc.copy()
    rng = np.random.Generator(np.random.PCG64(8))
    B, Nq, M, L, K = w.attn_weight.shape
    for l in range(L):
        H, W = w.spatial_shapes[l]
        far_lo_x = rng.uniform(-2.0, -0.5 / W - 1e-3, (B, Nq, M, K))
        far_hi_y = rng.uniform(1 + 0.5 / H + 1e-3, 3.0, (B, Nq, M, K))
        inside = rng.uniform(0.2, 0.8, (B, Nq, M, K))
        pick = rng.integers(0, 2, (B, Nq, M, K)).astype(bool)
        loc[:, :, :, l, :, 0] = np.where(pick, far_lo_x, inside)
        loc[:, :, :, l, :, 1] = np.where(pick, inside, far_hi_y)
    o = _fwd(orc, w, sampling_loc=loc)
    assert np.all(o == 0.0)
    gv, gl, ga = _bwd(orc, w, sampling_loc=loc)
    assert np.all(gv == 0.0) and np.all(gl == 0.0) and np.all(ga == 0.0)
    # just inside the border a neighbour still contributes
    loc2 = np.full_like(loc, 0.5)
    loc2[..., 0] = -0.5 / 6 + 1e-3
    o = _fwd(orc, w, sampling_loc=loc2)
    assert np.any(o != 0.0)


def pin_nonfinite(orc):
    """NaN and +-Inf coordinates fall outside every pixel test: the point
    contributes zero and gets zero gradients (a reading: the pages do not
    cover non-finite coordinates)."""
    w = workloads.random_case(81, 1, ((4, 4),), 3, 1, 2, 4)
    loc = w.sampling_loc.copy()
    loc[0, 0, 0, 0, 0, 0] = np.nan
    loc[0, 1, 0, 0, 1, 1] = np.inf
    loc[0, 2, 0, 0, 2, 0] = -np.inf
    keep = np.ones_like(w.attn_weight)
    keep[0, 0, 0, 0, 0] = 0
    keep[0, 1, 0, 0, 1] = 0
    keep[0, 2, 0, 0, 2] = 0
    o = _fwd(orc, w, sampling_loc=loc)
    o_ref = _fwd(orc, w, attn_weight=w.attn_weight * keep)
    assert np.all(np.isfinite(o)) and max_rel(o, o_ref) < 1e-15
    gv, gl, ga = _bwd(orc, w, sampling_loc=loc)
    assert np.all(np.isfinite(gl)) and np.all(np.isfinite(ga)) and np.all(np.isfinite(gv))
    for idx in ((0, 0, 0, 0, 0), (0, 1, 0, 0, 1), (0, 2, 0, 0, 2)):
        assert ga[idx] == 0.0 and np.all(gl[idx] == 0.0)


def pin_linearity(orc):
    """The output is a weighted sum: F(A1 + A2) = F(A1) + F(A2), F(sA) = sF(A)."""
    w = workloads.random_case(91, 1, ((5, 5), (2, 3)), 6, 2, 4, 2)
    rng = np.random.Generator(np.random.PCG64(4))
    a1 = rng.standard_normal(w.attn_weight.shape).astype(np.float32)
    a2 = rng.standard_normal(w.attn_weight.shape).astype(np.float32)
    f1 = _fwd(orc, w, mode=oracle.DOUBLE, attn_weight=a1)
    f2 = _fwd(orc, w, mode=oracle.DOUBLE, attn_weight=a2)
    f12 = _fwd(orc, w, mode=oracle.DOUBLE, attn_weight=(a1.astype(np.float64) + a2).astype(np.float32))
    assert max_rel(f12, f1 + f2) < 1e-6
    f3 = _fwd(orc, w, mode=oracle.DOUBLE, attn_weight=a1 * np.float32(2.0))
    assert max_rel(f3, 2.0 * f1) < 1e-15


# ----------------------------------------------------------------------------
# The other pixel convention, x = u*(W-1) (grid_sample align_corners=True),
# which the first page, section 2.3, advises offering as a configuration.
# ----------------------------------------------------------------------------
def pin_align_corners_grid_sample(orc):
    """In align-corners mode the forward and all three gradients equal the
    grid_sample composition with align_corners=True (torch CPU, fp64),
    including maps one pixel wide or tall and points beyond the border."""
    cases = [workloads.random_case(61, 2, ((5, 7), (3, 4), (2, 1)), 9, 3, 4, 3),
             workloads.random_case(62, 1, ((6, 6),), 7, 1, 2, 5, -0.6, 1.6),
             workloads.random_case(63, 2, ((1, 9), (4, 1)), 5, 2, 3, 2)]
    mode = oracle.DOUBLE | oracle.ALIGN
    for w in cases:
        out, gv, gl, ga = torch_reference(w, align_corners=True)
        o = _fwd(orc, w, mode=mode)
        assert max_rel(o, out) < 1e-12, f"align forward vs grid_sample on {w.name}"
        v, l_, a = _bwd(orc, w, mode=mode)
        assert max_rel(v, gv) < 1e-12, f"align grad_value vs autograd on {w.name}"
        assert max_rel(l_, gl) < 1e-9, f"align grad_loc vs autograd on {w.name}"
        assert max_rel(a, ga) < 1e-12, f"align grad_attn vs autograd on {w.name}"


def pin_align_corner_pixels(orc):
    """In align-corners mode the location (j/(W-1), i/(H-1)) is pixel (i, j)
    itself: the sample is value[i, j] (exactly in fp64; within 1e-6 in the fp32
    spec mode, whose product can land just below the integer).  Along an axis
    of one pixel every location maps to that pixel."""
    w = workloads.random_case(71, 2, ((5, 7), (3, 2), (1, 4), (6, 1)), 12, 3, 8, 2)
    B, Nq, M, L, K = w.attn_weight.shape
    rng = np.random.Generator(np.random.PCG64(6))
    loc = w.sampling_loc.copy()
    attn = np.zeros_like(w.attn_weight)
    expect = np.zeros((B, Nq, M, 8))
    for b in range(B):
        for q in range(Nq):
            for m in range(M):
                l = int(rng.integers(L))
                k = int(rng.integers(K))
                H, W = w.spatial_shapes[l]
                i, j = int(rng.integers(H)), int(rng.integers(W))
                u = j / (W - 1) if W > 1 else float(rng.uniform(0, 1))
                v = i / (H - 1) if H > 1 else float(rng.uniform(0, 1))
                loc[b, q, m, l, k] = (np.float32(u), np.float32(v))
                attn[b, q, m, l, k] = 1.0
                expect[b, q, m] = w.value[b, w.level_start_index[l] + i * W + j, m]
    for mode, tol in ((oracle.DOUBLE | oracle.ALIGN, 1e-6), (oracle.SPEC | oracle.ALIGN, 1e-6)):
        got = _fwd(orc, w, mode=mode, sampling_loc=loc, attn_weight=attn).reshape(B, Nq, M, 8)
        err = float(np.max(np.abs(got - expect)))
        assert err <= tol, f"align-corners pixel sample off by {err} (mode {mode})"


def pin_align_finite_differences(orc):
    """Central differences of the fp64 align-corners forward match its
    backward: d x / d u = W - 1 (points near a cell edge skipped)."""
    w = workloads.random_case(81, 1, ((5, 6), (3, 4)), 6, 2, 4, 2, 0.05, 0.95)
    mode = oracle.DOUBLE | oracle.ALIGN
    _, gl, _ = _bwd(orc, w, mode=mode)
    g = w.grad_out.astype(np.float64)

    def obj(**over):
        return float(np.sum(_fwd(orc, w, mode=mode, **over) * g))

    B, Nq, M, L, K = w.attn_weight.shape
    checked = 0
    rng = np.random.Generator(np.random.PCG64(8))
    for _ in range(40):
        b, q, m, l, k = (int(rng.integers(n)) for n in (B, Nq, M, L, K))
        H, W = w.spatial_shapes[l]
        for c, n in ((0, W), (1, H)):
            u = float(w.sampling_loc[b, q, m, l, k, c])
            p = u * (n - 1)
            h = 1e-3 / n
            if abs(p - np.round(p)) < 4e-3:
                continue
            lp = w.sampling_loc.copy()
            lm = w.sampling_loc.copy()
            lp[b, q, m, l, k, c] = u + h
            lm[b, q, m, l, k, c] = u - h
            hh = float(lp[b, q, m, l, k, c]) - float(lm[b, q, m, l, k, c])
            fd = (obj(sampling_loc=lp) - obj(sampling_loc=lm)) / hh
            an = gl[b, q, m, l, k, c]
            assert abs(fd - an) <= 1e-4 * max(1.0, abs(an)), f"align grad_loc fd {fd} vs {an}"
            checked += 1
    assert checked >= 20


ALL_PINS = [pin_pixel_centres, pin_one_hot_grid_sample, pin_four_point_example,
            pin_zero_offsets, pin_finite_differences, pin_adjoint,
            pin_partition_of_unity, pin_out_of_map, pin_nonfinite, pin_linearity,
            pin_align_corners_grid_sample, pin_align_corner_pixels,
            pin_align_finite_differences]
