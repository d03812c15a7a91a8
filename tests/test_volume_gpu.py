"""GPU parity of the 3-D (trilinear) variant (msda3d_forward, msda3d_backward)
against the CPU oracle (oracle/msda3d_oracle.c).  Metric and bars as the 2-D
core: max|x - r| / max|r|, fp32 forward 1e-5, backward 1e-4 (grad_value is
summed with atomics in no fixed order); bf16 value against the oracle on the
bf16-rounded values at the fp32 bars."""
import numpy as np
import pytest
import torch

import oracle
import oracle.volume as ov
import workloads
from oracle_pins import max_rel

pytestmark = pytest.mark.gpu

FWD_TOL = 1e-5
BWD_TOL = 1e-4


@pytest.fixture(scope="module")
def msda():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests must run on an MI355X")
    import scale_deformable_attention_04_amd as m
    m.load()
    return m


def _say(msg):
    print(f"[case] {msg}", flush=True)


def dev_inputs(w, bf16=False):
    d = torch.device("cuda:0")
    if bf16:
        value = torch.from_numpy(w.value_bf16.view(np.int16).copy()).view(torch.bfloat16).to(d)
    else:
        value = torch.from_numpy(w.value).to(d)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(d)
    return dict(value=value, volume_shapes=t(w.spatial_shapes),
                level_start_index=t(w.level_start_index), sampling_loc=t(w.sampling_loc),
                attn_weight=t(w.attn_weight))


def _args(w, loc=None, attn=None):
    return (w.value, w.spatial_shapes, w.level_start_index,
            w.sampling_loc if loc is None else loc, w.attn_weight if attn is None else attn)


def check(m, w, bf16=False, align=False, backward=True):
    x = dev_inputs(w, bf16)
    mode = oracle.SPEC | (oracle.ALIGN if align else 0)
    out = m.forward3d(**x, align_corners=align)
    torch.cuda.synchronize()
    e = max_rel(out.cpu().numpy(), ov.forward(*_args(w), mode=mode).reshape(out.shape))
    assert e <= FWD_TOL, f"{w.name}: forward max rel {e:.3e}"
    if not backward:
        return
    g = torch.from_numpy(w.grad_out).cuda()
    gv, gl, ga = m.backward3d(**x, grad_out=g, align_corners=align)
    torch.cuda.synchronize()
    rv, rl, ra = ov.backward(*_args(w), w.grad_out, mode=mode)
    for name, a, r in (("grad_value", gv, rv), ("grad_sampling_loc", gl, rl),
                       ("grad_attn_weight", ga, ra)):
        e = max_rel(a.cpu().numpy(), r)
        assert e <= BWD_TOL, f"{w.name}: {name} max rel {e:.3e}"


SHAPES = ((5, 9, 11), (3, 4, 6), (1, 3, 2))


@pytest.mark.parametrize("D", [4, 8, 16, 32, 64, 128, 256])
def test_volume_random_shapes(msda, D):
    _say(f"volume D={D}")
    w = workloads.volume_case(2000 + D, 2, SHAPES, 23, 2, D, 3)
    check(msda, w)


@pytest.mark.parametrize("L,K", [(1, 1), (1, 9), (3, 5), (4, 8)])
def test_volume_point_counts(msda, L, K):
    _say(f"volume L={L} K={K}")
    shapes = ((4, 6, 5), (2, 3, 3), (1, 2, 2), (2, 1, 7))[:L]
    w = workloads.volume_case(2100 + L + K, 2, shapes, 17, 3, 32, K)
    check(msda, w)


@pytest.mark.parametrize("D", [32, 64])
def test_volume_bf16(msda, D):
    _say(f"volume bf16 D={D}")
    w = workloads.volume_case(2200 + D, 2, SHAPES, 19, 2, D, 4, bf16=True)
    check(msda, w, bf16=True)


@pytest.mark.parametrize("D", [8, 32])
def test_volume_align_corners(msda, D):
    _say(f"volume align D={D}")
    w = workloads.volume_case(2300 + D, 2, SHAPES, 21, 2, D, 3, loc_low=-0.2, loc_high=1.2)
    check(msda, w, align=True)


def test_volume_out_of_volume_and_nonfinite(msda):
    _say("volume out of volume / non-finite")
    w = workloads.volume_case(2401, 1, SHAPES, 13, 2, 16, 3)
    loc = w.sampling_loc.copy()
    loc[0, 0, :, :, :, 2] = 1.6             # beyond the top face of every level
    loc[0, 1, :, :, 0, 0] = np.nan
    loc[0, 2, :, :, 1, 1] = np.inf
    loc[0, 3, :, :, 2, 2] = -np.inf
    loc[0, 4, 0, 0, 0, :] = -3.0            # far outside on every axis
    w.sampling_loc = loc
    check(msda, w)


@pytest.mark.parametrize("i", range(16))
def test_volume_sweep(msda, i):
    # seeded random volumes: 1-3 levels of up to 6 x 12 x 12, every head
    # width, 1..6 points, fp32 or bf16 value, either convention
    rng = np.random.Generator(np.random.PCG64(9800 + i))
    L = int(rng.integers(1, 4))
    shapes = tuple((int(rng.integers(1, 7)), int(rng.integers(1, 13)), int(rng.integers(1, 13)))
                   for _ in range(L))
    D = int(rng.choice([4, 8, 16, 32, 64, 128, 256]))
    B, Nq, M, K = (int(rng.integers(1, 3)), int(rng.integers(1, 60)), int(rng.integers(1, 5)),
                   int(rng.integers(1, 7)))
    bf16, align = bool(rng.integers(2)), bool(rng.integers(2))
    _say(f"volume sweep {i}: shapes={shapes} B={B} Nq={Nq} M={M} D={D} K={K} bf16={bf16} "
         f"align={align}")
    w = workloads.volume_case(9900 + i, B, shapes, Nq, M, D, K, bf16=bf16,
                              loc_low=-0.15, loc_high=1.15)
    check(msda, w, bf16=bf16, align=align)


def test_volume_empty(msda):
    _say("volume empty")
    w = workloads.volume_case(2501, 2, SHAPES, 0, 2, 8, 3)
    x = dev_inputs(w)
    out = msda.forward3d(**x)
    assert out.shape == (2, 0, 16)
    gv, gl, ga = msda.backward3d(**x, grad_out=torch.zeros(2, 0, 16, device="cuda"))
    torch.cuda.synchronize()
    assert float(gv.abs().max()) == 0.0 and gl.numel() == 0 and ga.numel() == 0


def test_volume_accumulate_and_autograd(msda):
    _say("volume accumulate, autograd")
    w = workloads.volume_case(2601, 1, SHAPES, 15, 2, 8, 3)
    x = dev_inputs(w)
    g = torch.from_numpy(w.grad_out).cuda()
    base = torch.randn(tuple(w.value.shape), generator=torch.Generator().manual_seed(4)).cuda()
    gv = base.clone()
    msda.backward3d(**x, grad_out=g, grad_value=gv, accumulate=True)
    torch.cuda.synchronize()
    rv, rl, ra = ov.backward(*_args(w), w.grad_out)
    assert max_rel(gv.cpu().numpy(), base.cpu().numpy() + rv) <= BWD_TOL
    leaves = {k: x[k].clone().requires_grad_(True)
              for k in ("value", "sampling_loc", "attn_weight")}
    out = msda.ms_deform_attn_3d(leaves["value"], x["volume_shapes"], x["level_start_index"],
                                 leaves["sampling_loc"], leaves["attn_weight"])
    out.backward(g)
    torch.cuda.synchronize()
    for name, r in (("value", rv), ("sampling_loc", rl), ("attn_weight", ra)):
        assert max_rel(leaves[name].grad.cpu().numpy(), r) <= BWD_TOL, name


@pytest.mark.parametrize("D", [32, 64])
def test_volume_split_bins(msda, D):
    # one 1x5x6 level: a single plane tile takes ~1500 x 4 points' records
    # per head, split over several items (partial tiles combined at D = 32,
    # atomic adds into zeroed tiles at D = 64); overwrite mode from NaN
    w = workloads.volume_case(2700 + D, 2, ((1, 5, 6), (2, 8, 9)), 1500, 2, D, 4)
    x = dev_inputs(w)
    g = torch.from_numpy(w.grad_out).cuda()
    _say(f"volume split bins D={D}")
    gv0 = torch.full(tuple(w.value.shape), float("nan"), device="cuda")
    gv, gl, ga = msda.backward3d(**x, grad_out=g, grad_value=gv0)
    torch.cuda.synchronize()
    rv, rl, ra = ov.backward(*_args(w), w.grad_out, mode=oracle.SPEC)
    got = gv.cpu().numpy()
    assert np.all(np.isfinite(got))
    for name, a, r in (("grad_value", got, rv), ("grad_sampling_loc", gl.cpu().numpy(), rl),
                       ("grad_attn_weight", ga.cpu().numpy(), ra)):
        e = max_rel(a, r)
        assert e <= BWD_TOL, f"{w.name}: {name} max rel {e:.3e}"


@pytest.mark.parametrize("D", [32, 64])
def test_volume_in_passes(msda, D):
    # the smallest workspace (msda3d_backward_workspace_min): grad_value in
    # passes of 1024 queries of one head of one batch (1500 = 1024 + 476;
    # 2 batches x 2 heads); overwrite mode from NaN
    w = workloads.volume_case(2800 + D, 2, ((1, 5, 6), (2, 8, 9)), 1500, 2, D, 4)
    B, Nv, Nq, M, _, L, K = (w.dims[k] for k in ("B", "Nv", "Nq", "M", "D", "L", "K"))
    least = msda.workspace_min3d(B, Nv, Nq, M, D, L, K)
    assert least < msda.workspace_size3d(B, Nv, Nq, M, D, L, K)
    x = dev_inputs(w)
    g = torch.from_numpy(w.grad_out).cuda()
    _say(f"volume in passes D={D}, workspace {least} bytes")
    gv0 = torch.full(tuple(w.value.shape), float("nan"), device="cuda")
    gv, gl, ga = msda.backward3d(**x, grad_out=g, grad_value=gv0,
                                 workspace=torch.empty(least, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    rv, rl, ra = ov.backward(*_args(w), w.grad_out, mode=oracle.SPEC)
    for name, a, r in (("grad_value", gv.cpu().numpy(), rv),
                       ("grad_sampling_loc", gl.cpu().numpy(), rl),
                       ("grad_attn_weight", ga.cpu().numpy(), ra)):
        e = max_rel(a, r)
        assert e <= BWD_TOL, f"{w.name}: {name} max rel {e:.3e}"


def test_volume_workload(msda):
    # the voxel workload: pyramid 4x128x128, 2x64x64, 1x32x32, 16,384 bird's-eye
    # queries, M=8, D=32, K=4, forward and backward in full
    _say("volume workload B=1 Nq=16384 M=8 D=32 L=3 K=4")
    check(msda, workloads.make_volume())
