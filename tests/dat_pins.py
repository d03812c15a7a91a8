"""Pins for the DAT oracle (oracle/dat.py).

Each ``pin_*`` takes the module under test (``oracle.dat`` or a copy with a
planted mistake) and raises AssertionError when it disagrees with what the
pages or the mathematics fix:

  pin_dat_sdpa              torch CPU fp64 scaled_dot_product_attention with the
                            bias as an additive mask: forward, and autograd
                            gradients of q, k, v and the bias
  pin_dat_uniform           zero queries and no bias give uniform weights: each
                            output is the mean of the values; a bias that
                            leaves one key per row finite selects that value
  pin_dat_row_shift         adding a constant to a row of the bias changes
                            nothing, and each row of the bias gradient sums to 0
  pin_dat_finite_differences central differences of the fp64 forward
  pin_dat_sampling          the sampling step equals the page's own
                            grid_sample(bilinear, align_corners=True) per group
                            (DAT integration page, section 2.2), forward and
                            autograd backward
"""
from __future__ import annotations

import numpy as np
import torch
import torch.nn.functional as F

import oracle
import workloads
from oracle_pins import max_rel


def _case(seed=1, with_bias=True, N_hw=(5, 4), Ns_hw=(3, 2)):
    return workloads.dat_case(seed, 2, N_hw[0], N_hw[1], 24, 3, 2, Ns_hw[0], Ns_hw[1],
                              with_bias=with_bias)


def pin_dat_sdpa(impl):
    for with_bias in (True, False):
        w = _case(11 + with_bias, with_bias=with_bias)
        t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
        q, k, v = t(w.q), t(w.k), t(w.v)
        bias = t(w.bias) if with_bias else None
        # torch's layout [B, heads, tokens, d]
        o = F.scaled_dot_product_attention(q.permute(0, 2, 1, 3), k.permute(0, 2, 1, 3),
                                           v.permute(0, 2, 1, 3), attn_mask=bias)
        o = o.permute(0, 2, 1, 3)
        o.backward(torch.tensor(w.grad_out, dtype=torch.float64))
        out, lse = impl.attention(w.q, w.k, w.v, w.bias if with_bias else None)
        dq, dk, dv, db = impl.attention_backward(w.q, w.k, w.v, w.grad_out,
                                                 w.bias if with_bias else None)
        assert max_rel(out, o.detach().numpy()) < 1e-12
        assert max_rel(dq, q.grad.numpy()) < 1e-12
        assert max_rel(dk, k.grad.numpy()) < 1e-12
        assert max_rel(dv, v.grad.numpy()) < 1e-12
        if with_bias:
            assert max_rel(db, bias.grad.numpy()) < 1e-12
        # lse is the log of the softmax denominator of each row
        s = np.einsum("bnhd,bshd->bhns", w.q.astype(np.float64), w.k) / np.sqrt(w.q.shape[-1])
        if with_bias:
            s = s + w.bias
        assert max_rel(lse, np.log(np.exp(s).sum(-1))) < 1e-12


def pin_dat_uniform(impl):
    w = _case(21, with_bias=False)
    zq = np.zeros_like(w.q)
    out, _ = impl.attention(zq, w.k, w.v, None)
    mean_v = w.v.astype(np.float64).mean(axis=1)                    # [B, heads, d]
    assert max_rel(out, np.broadcast_to(mean_v[:, None], out.shape)) < 1e-12
    B, N, Hh, _ = w.q.shape
    Ns = w.k.shape[1]
    pick = np.random.Generator(np.random.PCG64(4)).integers(0, Ns, (B, Hh, N))
    bias = np.full((B, Hh, N, Ns), -1e30)
    np.put_along_axis(bias, pick[..., None], 0.0, axis=-1)
    out, _ = impl.attention(w.q, w.k, w.v, bias)
    want = np.take_along_axis(w.v.transpose(0, 2, 1, 3)[:, :, None],      # [B, Hh, 1, Ns, d]
                              pick[..., None, None], axis=3)[:, :, :, 0]  # [B, Hh, N, d]
    assert max_rel(out, want.transpose(0, 2, 1, 3)) < 1e-12


def pin_dat_row_shift(impl):
    w = _case(31)
    B, N, Hh, _ = w.q.shape
    c = np.random.Generator(np.random.PCG64(5)).integers(-3, 4, (B, Hh, N, 1)).astype(np.float64)
    a, _ = impl.attention(w.q, w.k, w.v, w.bias)
    b, _ = impl.attention(w.q, w.k, w.v, w.bias.astype(np.float64) + c)
    assert max_rel(b, a) < 1e-12
    _, _, _, db = impl.attention_backward(w.q, w.k, w.v, w.grad_out, w.bias)
    assert float(np.max(np.abs(db.sum(-1)))) < 1e-12 * float(np.max(np.abs(db))) * db.shape[-1]
    assert float(np.max(np.abs(db))) > 0


def pin_dat_finite_differences(impl):
    w = _case(41)
    g = w.grad_out.astype(np.float64)
    dq, dk, dv, db = impl.attention_backward(w.q, w.k, w.v, w.grad_out, w.bias)
    r = np.random.Generator(np.random.PCG64(6))
    args = {"q": w.q.astype(np.float64), "k": w.k.astype(np.float64),
            "v": w.v.astype(np.float64), "bias": w.bias.astype(np.float64)}
    grads = {"q": dq, "k": dk, "v": dv, "bias": db}

    def f(**over):
        a = dict(args)
        a.update(over)
        out, _ = impl.attention(a["q"], a["k"], a["v"], a["bias"])
        return float(np.sum(out * g))

    h = 1e-5
    for name in ("q", "k", "v", "bias"):
        d = r.standard_normal(args[name].shape)
        fd = (f(**{name: args[name] + h * d}) - f(**{name: args[name] - h * d})) / (2 * h)
        an = float(np.sum(grads[name] * d))
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def pin_dat_sampling(impl):
    # the page's step: grid_sample(x.reshape(B*G, Dg, H, W), pos in [-1, 1] as
    # (x, y), bilinear, align_corners=True), one sampled key per reference point
    w = _case(51)
    B, HW, G, Dg = w.x.shape
    H, W = w.hw
    Ns = w.pos.shape[1]
    x = torch.tensor(w.x, dtype=torch.float64, requires_grad=True)
    pos = torch.tensor(w.pos, dtype=torch.float64, requires_grad=True)
    xg = x.reshape(B, H, W, G, Dg).permute(0, 3, 4, 1, 2).reshape(B * G, Dg, H, W)
    grid = (2.0 * pos - 1.0).permute(0, 2, 1, 3).reshape(B * G, 1, Ns, 2)
    smp = F.grid_sample(xg, grid, mode="bilinear", padding_mode="zeros", align_corners=True)
    smp = smp.reshape(B, G, Dg, Ns).permute(0, 3, 1, 2).reshape(B, Ns, G * Dg)
    smp.backward(torch.tensor(w.grad_sampled, dtype=torch.float64))
    got = impl.sample(w.x, w.hw, w.pos, mode=oracle.DOUBLE)
    gx, gp = impl.sample_backward(w.x, w.hw, w.pos, w.grad_sampled, mode=oracle.DOUBLE)
    assert max_rel(got, smp.detach().numpy()) < 1e-12
    assert max_rel(gx, x.grad.numpy()) < 1e-12
    assert max_rel(gp, pos.grad.numpy()) < 1e-10


ALL_DAT_PINS = [pin_dat_sdpa, pin_dat_uniform, pin_dat_row_shift, pin_dat_finite_differences,
                pin_dat_sampling]
