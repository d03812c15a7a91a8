"""GPU parity of the fused prologue entry points (msda_forward_fused,
msda_backward_fused) against the CPU oracle (oracle/fused.py on top of the
core oracle).  Same metric and bars as the core: max|x - r| / max|r|, fp32
forward 1e-5, backward 1e-4; bf16 value compared with the oracle run on the
bf16-rounded values at the fp32 bars."""
import numpy as np
import pytest
import torch

import oracle
import oracle.fused as ofused
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


def dev_inputs(w: workloads.FusedWorkload, bf16=False):
    d = torch.device("cuda:0")
    if bf16:
        value = torch.from_numpy(w.value_bf16.view(np.int16).copy()).view(torch.bfloat16).to(d)
    else:
        value = torch.from_numpy(w.value).to(d)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(d)
    return dict(value=value, spatial_shapes=t(w.spatial_shapes),
                level_start_index=t(w.level_start_index), reference_points=t(w.reference_points),
                sampling_offsets=t(w.sampling_offsets), attn_logits=t(w.attn_logits))


def _mode(align):
    return oracle.SPEC | (oracle.ALIGN if align else 0)


def _oracle_args(w):
    return (w.value, w.spatial_shapes, w.level_start_index, w.reference_points,
            w.sampling_offsets, w.attn_logits)


def check(m, w, per_level=False, align=False, bf16=False, backward=True, need_grad_ref=True,
          saved=False):
    """Forward and backward against the oracle; with w.attn_scale set, the
    scale attention and its gradient too; saved=True hands the forward's
    locations and weights to the backward."""
    x = dev_inputs(w, bf16)
    S = w.attn_scale
    sx = {} if S is None else {"scale": torch.from_numpy(S).cuda()}
    res = m.forward_fused(**x, per_level=per_level, align_corners=align, save=saved, **sx)
    out = res[0] if saved else res
    torch.cuda.synchronize()
    r_out = ofused.forward(*_oracle_args(w), per_level=per_level, mode=_mode(align), scale=S)
    e = max_rel(out.cpu().numpy(), r_out.reshape(out.shape))
    assert e <= FWD_TOL, f"{w.name}: fused forward max rel {e:.3e}"
    if not backward:
        return
    g = torch.from_numpy(w.grad_out).cuda()
    res = m.backward_fused(**x, grad_out=g, per_level=per_level, align_corners=align,
                           need_grad_ref=need_grad_ref, saved=tuple(res[1:]) if saved else None,
                           **sx)
    torch.cuda.synchronize()
    ref = ofused.backward(*_oracle_args(w), w.grad_out, per_level=per_level, mode=_mode(align),
                          scale=S)
    assert len(res) == len(ref)
    gv, goff, gz, gref = res[:4]
    rv, roff, rz, rref = ref[:4]
    got = [("grad_value", gv, rv), ("grad_sampling_offsets", goff, roff),
           ("grad_attn_logits", gz, rz)]
    if S is not None:
        got.append(("grad_scale", res[4], ref[4]))
    if need_grad_ref:
        got.append(("grad_reference_points", gref, rref))
    else:
        assert gref is None
    for name, a, r in got:
        e = max_rel(a.cpu().numpy(), r)
        assert e <= BWD_TOL, f"{w.name}: {name} max rel {e:.3e}"


SHAPES = ((13, 17), (7, 9), (3, 4))


@pytest.mark.parametrize("D", [4, 8, 16, 32, 64, 256])
@pytest.mark.parametrize("per_level", [False, True])
def test_fused_random_shapes(msda, D, per_level):
    _say(f"fused D={D} per_level={per_level}")
    w = workloads.fused_case(100 + D, 2, SHAPES, 37, 3, D, 3, ref_low=-0.05, ref_high=1.05)
    check(msda, w, per_level=per_level)


# power-of-two softmax groups of at most 64 points are reduced with lane
# shuffles (when the forward's point table holds whole items); the others, as
# in the cases above (L*K = 9 or 15), with per-group statistics in LDS
@pytest.mark.parametrize("D,L,K", [(16, 4, 4), (64, 2, 32), (64, 1, 64), (32, 2, 8), (8, 4, 16),
                                   (32, 1, 1)])
@pytest.mark.parametrize("per_level", [False, True])
def test_fused_shuffle_groups(msda, D, L, K, per_level):
    _say(f"fused groups D={D} L={L} K={K} per_level={per_level}")
    shapes = ((11, 13), (6, 5), (4, 3), (2, 2))[:L]
    w = workloads.fused_case(1000 + D + L + K, 2, shapes, 27, 2, D, K, ref_low=-0.05,
                             ref_high=1.05)
    check(msda, w, per_level=per_level)


@pytest.mark.parametrize("per_level,align", [(False, True), (True, True)])
def test_fused_align_corners(msda, per_level, align):
    _say(f"fused align per_level={per_level}")
    w = workloads.fused_case(201, 2, SHAPES, 29, 2, 32, 4)
    check(msda, w, per_level=per_level, align=align)


@pytest.mark.parametrize("per_level", [False, True])
def test_fused_bf16(msda, per_level):
    _say(f"fused bf16 per_level={per_level}")
    w = workloads.fused_case(301, 2, SHAPES, 41, 4, 32, 4, bf16=True)
    check(msda, w, per_level=per_level, bf16=True)


def test_fused_large_logits_and_no_ref_grad(msda):
    # logits N(0, 30): the softmax must subtract its maximum
    _say("fused large logits, grad_ref not requested")
    w = workloads.fused_case(401, 1, SHAPES, 23, 2, 16, 5, logit_scale=30.0)
    check(msda, w, per_level=False, need_grad_ref=False)
    check(msda, w, per_level=True)


def test_fused_sixteen_levels_small_head(msda):
    # D = 4: 256 items per workgroup, the point tables are processed in chunks
    # of one point next to the per-level softmax statistics
    _say("fused L=16 D=4 per_level")
    shapes = tuple((1 + (l % 5), 2 + (l % 3)) for l in range(16))
    w = workloads.fused_case(501, 2, shapes, 19, 2, 4, 2)
    check(msda, w, per_level=True)
    check(msda, w, per_level=False)


@pytest.mark.parametrize("D,K,per_level", [(32, 4, False), (4, 2, True), (16, 3, False)])
def test_fused_saved_locations(msda, D, K, per_level):
    # forward_fused(save=True) stores the locations -- bit for bit the fp32
    # division and addition of the oracle -- and the weights; the backward
    # reading them gives the same gradients as the one recomputing them
    _say(f"fused saved locations D={D} K={K} per_level={per_level}")
    w = workloads.fused_case(1101 + D, 2, SHAPES, 31, 2, D, K, ref_low=-0.05, ref_high=1.05)
    x = dev_inputs(w)
    out, loc, attn = msda.forward_fused(**x, per_level=per_level, save=True)
    torch.cuda.synchronize()
    r_loc = ofused.locations(w.reference_points, w.sampling_offsets, w.spatial_shapes)
    assert np.array_equal(loc.cpu().numpy().view(np.uint32), r_loc.view(np.uint32))
    r_attn = ofused.weights(w.attn_logits, SHAPES.__len__(), K, per_level)
    assert float(np.max(np.abs(attn.cpu().numpy() - r_attn))) <= 1e-6
    plain = msda.forward_fused(**x, per_level=per_level)
    assert torch.equal(out, plain)
    g = torch.from_numpy(w.grad_out).cuda()
    a = msda.backward_fused(**x, grad_out=g, per_level=per_level, saved=(loc, attn))
    torch.cuda.synchronize()
    rv, roff, rz, rref = ofused.backward(*_oracle_args(w), w.grad_out, per_level=per_level)
    for name, got, r in zip(("grad_value", "grad_offsets", "grad_logits", "grad_ref"), a,
                            (rv, roff, rz, rref)):
        e = max_rel(got.cpu().numpy(), r)
        assert e <= BWD_TOL, f"{name}: {e:.3e}"


def test_fused_accumulate(msda):
    _say("fused accumulate")
    w = workloads.fused_case(601, 1, SHAPES, 17, 2, 8, 3)
    x = dev_inputs(w)
    g = torch.from_numpy(w.grad_out).cuda()
    base = torch.randn(tuple(w.value.shape), generator=torch.Generator().manual_seed(3)).cuda()
    gv = base.clone()
    msda.backward_fused(**x, grad_out=g, grad_value=gv, accumulate=True)
    torch.cuda.synchronize()
    rv, _, _, _ = ofused.backward(*_oracle_args(w), w.grad_out)
    e = max_rel(gv.cpu().numpy(), base.cpu().numpy() + rv)
    assert e <= BWD_TOL


@pytest.mark.parametrize("acc", [False, True])
def test_fused_in_passes(msda, acc):
    """The smallest fused workspace: grad_value in passes of 1024 queries of
    one head of one batch (1500 = 1024 + 476; 2 batches x 2 heads), the
    other gradients as ever."""
    w = workloads.fused_case(611, 2, SHAPES, 1500, 2, 16, 4)
    B, Nv, Nq, M, D, L, K = (w.dims[k] for k in ("B", "Nv", "Nq", "M", "D", "L", "K"))
    least = msda.fused_workspace_min(B, Nv, Nq, M, D, L, K)
    assert least < msda.fused_workspace_size(B, Nv, Nq, M, D, L, K)
    _say(f"fused in passes acc={acc}, workspace {least} bytes")
    x = dev_inputs(w)
    g = torch.from_numpy(w.grad_out).cuda()
    base = torch.randn(tuple(w.value.shape), generator=torch.Generator().manual_seed(4)).cuda()
    gv0 = base.clone() if acc else torch.full(tuple(w.value.shape), float("nan"), device="cuda")
    res = msda.backward_fused(**x, grad_out=g, grad_value=gv0, accumulate=acc,
                              workspace=torch.empty(least, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    ref = ofused.backward(*_oracle_args(w), w.grad_out)
    got_v = res[0].cpu().numpy() - (base.cpu().numpy() if acc else 0.0)
    for name, a, r in (("grad_value", got_v, ref[0]),
                       ("grad_sampling_offsets", res[1].cpu().numpy(), ref[1]),
                       ("grad_attn_logits", res[2].cpu().numpy(), ref[2]),
                       ("grad_reference_points", res[3].cpu().numpy(), ref[3])):
        e = max_rel(a, r)
        assert e <= BWD_TOL, f"{name} max rel {e:.3e}"


def test_fused_empty(msda):
    _say("fused empty")
    w = workloads.fused_case(701, 1, SHAPES, 0, 2, 8, 3)
    x = dev_inputs(w)
    out = msda.forward_fused(**x)
    assert out.shape == (1, 0, 16)
    g = torch.zeros((1, 0, 16), device="cuda")
    gv, goff, gz, gref = msda.backward_fused(**x, grad_out=g)
    torch.cuda.synchronize()
    assert float(gv.abs().max()) == 0.0 and goff.numel() == 0 and gref.numel() == 0


def test_fused_autograd_function(msda):
    _say("fused autograd")
    w = workloads.fused_case(801, 2, SHAPES, 21, 2, 16, 3)
    x = dev_inputs(w)
    leaves = {k: x[k].clone().requires_grad_(True)
              for k in ("value", "reference_points", "sampling_offsets", "attn_logits")}
    out = msda.ms_deform_attn_fused(leaves["value"], x["spatial_shapes"],
                                    x["level_start_index"], leaves["reference_points"],
                                    leaves["sampling_offsets"], leaves["attn_logits"],
                                    per_level=True)
    out.backward(torch.from_numpy(w.grad_out).cuda())
    torch.cuda.synchronize()
    rv, roff, rz, rref = ofused.backward(*_oracle_args(w), w.grad_out, per_level=True)
    for name, r in (("value", rv), ("sampling_offsets", roff), ("attn_logits", rz),
                    ("reference_points", rref)):
        e = max_rel(leaves[name].grad.cpu().numpy(), r)
        assert e <= BWD_TOL, f"{name}: {e:.3e}"


def test_fused_stage_events(msda):
    _say("fused stage events")
    w = workloads.fused_case(901, 2, SHAPES, 33, 2, 32, 4)
    x = dev_inputs(w)
    g = torch.from_numpy(w.grad_out).cuda()
    ev = msda.make_events(fused=True)
    gv, goff, gz, gref = msda.backward_fused(**x, grad_out=g, events=ev)
    torch.cuda.synchronize()
    t = msda.stage_times(ev)
    assert len(t) == len(msda.BWD_FUSED_STAGES) and all(v is not None and v >= 0 for v in t)
    rv, roff, rz, rref = ofused.backward(*_oracle_args(w), w.grad_out)
    assert max_rel(gz.cpu().numpy(), rz) <= BWD_TOL


def test_fused_encoder(msda):
    # the encoder-shape workload (B=2, 22,223 queries on the DETR levels,
    # M=8, D=32, L=4, K=4) in the fused input form, forward and backward in full
    _say("fused encoder B=2 Nq=Nv=22223")
    w = workloads.make_fused(3)
    check(msda, w, per_level=False)


def test_fused_train_bf16_per_level(msda):
    # B=4, K=8, bf16 value; the per-level softmax of the first page's text
    _say("fused train_bf16 B=4 K=8 per_level")
    w = workloads.make_fused(4)
    check(msda, w, per_level=True, bf16=True)


# ---------------------------------------------------------------------------
# the scale attention S of the multi-scale formula (weights S * softmax)
# ---------------------------------------------------------------------------
# softmax groups of 16 or 32 points are finished in the dots kernel (lane
# shuffles); groups of 9 or 15 points, and items whose points span several
# table chunks (L*K = 64 at D = 64), in the epilogue kernel
@pytest.mark.parametrize("D,L,K", [(16, 4, 4), (32, 4, 8), (32, 3, 3), (8, 3, 5), (64, 2, 32)])
@pytest.mark.parametrize("per_level", [False, True])
def test_fused_scale_attention(msda, D, L, K, per_level):
    _say(f"fused scale attention D={D} L={L} K={K} per_level={per_level}")
    shapes = ((11, 13), (6, 5), (4, 3), (2, 2))[:L]
    w = workloads.fused_case(1100 + D + 7 * L + K, 2, shapes, 33, 3, D, K, ref_low=-0.05,
                             ref_high=1.05, with_scale=True)
    check(msda, w, per_level=per_level)


@pytest.mark.parametrize("per_level,align,bf16", [(False, False, False), (True, True, True)])
def test_fused_scale_saved_and_conventions(msda, per_level, align, bf16):
    _say(f"fused scale saved per_level={per_level} align={align} bf16={bf16}")
    w = workloads.fused_case(1201, 2, SHAPES, 41, 4, 32, 4, with_scale=True, bf16=bf16)
    check(msda, w, per_level=per_level, align=align, bf16=bf16, saved=True)
    check(msda, w, per_level=per_level, align=align, bf16=bf16, need_grad_ref=False)


def test_fused_scale_encoder(msda):
    # the encoder-shape workload with a scale attention, forward and backward
    _say("fused scale encoder B=2 Nq=Nv=22223")
    check(msda, workloads.make_fused(3, with_scale=True), saved=True)


def test_fused_scale_autograd(msda):
    _say("fused scale autograd")
    w = workloads.fused_case(1301, 2, SHAPES, 19, 2, 16, 4, with_scale=True)
    x = dev_inputs(w)
    leaves = {k: x[k].clone().requires_grad_(True)
              for k in ("value", "reference_points", "sampling_offsets", "attn_logits")}
    S = torch.from_numpy(w.attn_scale).cuda().requires_grad_(True)
    out = msda.ms_deform_attn_fused(leaves["value"], x["spatial_shapes"], x["level_start_index"],
                                    leaves["reference_points"], leaves["sampling_offsets"],
                                    leaves["attn_logits"], scale=S)
    out.backward(torch.from_numpy(w.grad_out).cuda())
    rv, roff, rz, rref, rs = ofused.backward(*_oracle_args(w), w.grad_out, scale=w.attn_scale)
    r_out = ofused.forward(*_oracle_args(w), scale=w.attn_scale)
    assert max_rel(out.detach().cpu().numpy(), r_out.reshape(out.shape)) <= FWD_TOL
    for name, t, r in (("value", leaves["value"].grad, rv),
                       ("sampling_offsets", leaves["sampling_offsets"].grad, roff),
                       ("attn_logits", leaves["attn_logits"].grad, rz),
                       ("reference_points", leaves["reference_points"].grad, rref),
                       ("scale", S.grad, rs)):
        e = max_rel(t.cpu().numpy(), r)
        assert e <= BWD_TOL, f"{name}: {e:.3e}"
