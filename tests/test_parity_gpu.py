"""GPU parity: the HIP library (through its C ABI) against the CPU oracle.

Metric (per output tensor): max_i |x_i - r_i| / max_i |r_i|.  Bars: fp32
forward 1e-5; fp32 backward 1e-4 (grad_value is summed with atomics in no
fixed order); bf16 value 2e-2 against the oracle on the unrounded fp32 values,
and the fp32 bars against the oracle on the bf16-rounded values.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle_pins import max_rel

pytestmark = pytest.mark.gpu

FWD_TOL = 1e-5
BWD_TOL = 1e-4
BF16_TOL = 2e-2


@pytest.fixture(scope="module")
def msda():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests must run on an MI355X")
    import scale_deformable_attention_04_amd as m
    m.load()
    return m


def close(x, r, tol, what=""):
    e = max_rel(x, r)
    assert e <= tol, f"{what}: max rel error {e:.3e} > {tol}"


def _say(msg):
    print(f"[case] {msg}", flush=True)


def dev_inputs(w: workloads.Workload, bf16: bool = False):
    d = torch.device("cuda:0")
    if bf16:
        bits = torch.from_numpy(w.value_bf16.view(np.int16).copy())
        value = bits.view(torch.bfloat16).to(d)
    else:
        value = torch.from_numpy(w.value).to(d)
    t = lambda a, dt=None: torch.from_numpy(np.ascontiguousarray(a)).to(d)
    return dict(value=value, spatial_shapes=t(w.spatial_shapes),
                level_start_index=t(w.level_start_index), sampling_loc=t(w.sampling_loc),
                attn_weight=t(w.attn_weight))


def gpu_forward(m, w, bf16=False):
    x = dev_inputs(w, bf16)
    out = m.forward(**x)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def gpu_backward(m, w, bf16=False, **kw):
    x = dev_inputs(w, bf16)
    g = torch.from_numpy(w.grad_out).cuda()
    gv, gl, ga = m.backward(**x, grad_out=g, **kw)
    torch.cuda.synchronize()
    return gv.cpu().numpy(), gl.cpu().numpy(), ga.cpu().numpy()


def oracle_fwd(w, value=None, mode=oracle.SPEC):
    return oracle.forward(w.value if value is None else value, w.spatial_shapes,
                          w.level_start_index, w.sampling_loc, w.attn_weight, mode=mode)


def oracle_bwd(w, value=None, mode=oracle.SPEC):
    return oracle.backward(w.value if value is None else value, w.spatial_shapes,
                           w.level_start_index, w.sampling_loc, w.attn_weight, w.grad_out,
                           mode=mode)


def check_fwd(m, w, tol=FWD_TOL, bf16=False):
    got = gpu_forward(m, w, bf16)
    ref = oracle_fwd(w).reshape(got.shape)
    e = max_rel(got, ref)
    assert e <= tol, f"{w.name}: forward max rel {e:.3e} > {tol}"
    return got, e


def check_bwd(m, w, tol=BWD_TOL, bf16=False):
    gv, gl, ga = gpu_backward(m, w, bf16)
    rv, rl, ra = oracle_bwd(w)
    errs = (max_rel(gv, rv), max_rel(gl, rl), max_rel(ga, ra))
    for name, e in zip(("grad_value", "grad_sampling_loc", "grad_attn_weight"), errs):
        assert e <= tol, f"{w.name}: {name} max rel {e:.3e} > {tol}"
    return errs


# ---------------------------------------------------------------------------
# the five configurations at full size
# ---------------------------------------------------------------------------
def test_tiny_fwd_bwd(msda):
    _say("tiny fwd+bwd")
    w = workloads.make(0)
    check_fwd(msda, w)
    check_bwd(msda, w)


def test_encoder_fwd(msda):
    _say("encoder fwd B=2 Nq=Nv=22223 M=8 D=32 L=4 K=4")
    check_fwd(msda, workloads.make(1))


def test_decoder_fwd(msda):
    _say("decoder fwd B=2 Nq=300")
    check_fwd(msda, workloads.make(2))


def test_encoder_bwd(msda):
    _say("encoder bwd B=2 Nq=Nv=22223")
    check_bwd(msda, workloads.make(3))


def test_decoder_bwd(msda):
    """The decoder shape's backward (300 object queries over the encoder's
    4-level value: 4,800 points per head, so the binned pipeline), fp32 and
    with a bf16 value."""
    _say("decoder bwd B=2 Nq=300 fp32")
    w = workloads.make(2)
    check_bwd(msda, w)
    _say("decoder bwd B=2 Nq=300 bf16 value")
    bits = workloads.bf16_bits(w.value)
    wb = workloads.Workload(w.name + " bf16", workloads.bf16_to_f32(bits).reshape(w.value.shape),
                            w.spatial_shapes, w.level_start_index, w.sampling_loc,
                            w.attn_weight, w.grad_out, value_bf16=bits.reshape(w.value.shape),
                            value_unrounded=w.value)
    gv, gl, ga = gpu_backward(msda, wb, bf16=True)
    for x, r in zip((gv, gl, ga), oracle_bwd(wb)):             # bf16-rounded value
        close(x, r, BWD_TOL)
    for x, r in zip((gv, gl, ga), oracle_bwd(wb, wb.value_unrounded)):  # pass/fail bar
        close(x, r, BF16_TOL)


def test_train_bf16_fwd_bwd(msda):
    _say("train bf16 B=4 K=8 fwd+bwd")
    w = workloads.make(4)
    # strict: against the oracle on the bf16-rounded values (w.value)
    got = gpu_forward(msda, w, bf16=True)
    close(got, oracle_fwd(w).reshape(got.shape), FWD_TOL)
    gv, gl, ga = gpu_backward(msda, w, bf16=True)
    rv, rl, ra = oracle_bwd(w)
    for x, r in ((gv, rv), (gl, rl), (ga, ra)):
        close(x, r, BWD_TOL)
    # pass/fail bar: against the oracle on the unrounded fp32 values
    close(got, oracle_fwd(w, w.value_unrounded).reshape(got.shape), BF16_TOL)
    rv, rl, ra = oracle_bwd(w, w.value_unrounded)
    for x, r in ((gv, rv), (gl, rl), (ga, ra)):
        close(x, r, BF16_TOL)


# ---------------------------------------------------------------------------
# every head width, both value dtypes, ragged tails, several tiles
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("D", [4, 8, 16, 32, 64, 128, 256])
@pytest.mark.parametrize("bf16", [False, True])
def test_random_shapes(msda, D, bf16):
    shapes = ((13, 21), (7, 11), (4, 6))
    Nq = 301 if D <= 32 else 97      # several workgroups and a partial last one
    w = workloads.random_case(100 + D, 3, shapes, Nq, 3, D, 3, bf16=bf16)
    _say(f"random D={D} bf16={bf16} Nq={Nq}")
    check_fwd(msda, w, bf16=bf16)
    check_bwd(msda, w, bf16=bf16)


@pytest.mark.parametrize("L,K", [(1, 1), (1, 7), (3, 5), (4, 16), (2, 40)])
def test_point_counts(msda, L, K):
    """L*K up to 80: the point tables are walked in several chunks."""
    shapes = ((9, 10), (5, 5), (3, 2), (2, 2))[:L]
    w = workloads.random_case(200 + 10 * L + K, 2, shapes, 67, 4, 32, K)
    _say(f"points L={L} K={K}")
    check_fwd(msda, w)
    check_bwd(msda, w)


def test_sixteen_levels_and_thin_maps(msda):
    shapes = tuple((1 + (i % 4), 1 + (7 * i) % 9) for i in range(16))
    w = workloads.random_case(300, 2, shapes, 45, 2, 16, 2, -0.3, 1.3)
    _say("16 levels")
    check_fwd(msda, w)
    check_bwd(msda, w)


def test_many_tiles_use_global_bin_counters(msda):
    """A 520x520 level has 65*65 = 4225 tiles of 8x8, more than the LDS bin
    histograms hold: counts and record slots then go through global atomics."""
    w = workloads.random_case(350, 1, ((520, 520), (3, 3)), 64, 2, 8, 3)
    _say("4225 tiles")
    check_fwd(msda, w)
    check_bwd(msda, w)


# ---------------------------------------------------------------------------
# the align_corners pixel convention (x = u*(W-1), y = v*(H-1))
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("D,bf16", [(8, False), (32, False), (32, True), (64, False)])
def test_align_corners(msda, D, bf16):
    shapes = ((9, 13), (5, 7), (1, 6), (4, 1))
    w = workloads.random_case(360 + D, 2, shapes, 83, 3, D, 3, -0.2, 1.2, bf16=bf16)
    _say(f"align_corners D={D} bf16={bf16}")
    x = dev_inputs(w, bf16)
    out = msda.forward(**x, align_corners=True)
    g = torch.from_numpy(w.grad_out).cuda()
    gv, gl, ga = msda.backward(**x, grad_out=g, align_corners=True)
    torch.cuda.synchronize()
    mode = oracle.SPEC | oracle.ALIGN
    close(out.cpu().numpy(), oracle_fwd(w, mode=mode).reshape(out.shape), FWD_TOL, "forward")
    rv, rl, ra = oracle_bwd(w, mode=mode)
    close(gv.cpu().numpy(), rv, BWD_TOL, "grad_value")
    close(gl.cpu().numpy(), rl, BWD_TOL, "grad_sampling_loc")
    close(ga.cpu().numpy(), ra, BWD_TOL, "grad_attn_weight")
    # the two conventions really differ on these inputs
    assert max_rel(out.cpu().numpy(), oracle_fwd(w).reshape(out.shape)) > 1e-3


def test_align_corners_encoder(msda):
    """The encoder shape, forward and backward, in the align_corners convention."""
    w = workloads.make(3)
    _say("align_corners encoder")
    x = dev_inputs(w)
    out = msda.forward(**x, align_corners=True)
    gv, gl, ga = msda.backward(**x, grad_out=torch.from_numpy(w.grad_out).cuda(),
                               align_corners=True)
    torch.cuda.synchronize()
    mode = oracle.SPEC | oracle.ALIGN
    close(out.cpu().numpy(), oracle_fwd(w, mode=mode).reshape(out.shape), FWD_TOL, "forward")
    rv, rl, ra = oracle_bwd(w, mode=mode)
    close(gv.cpu().numpy(), rv, BWD_TOL, "grad_value")
    close(gl.cpu().numpy(), rl, BWD_TOL, "grad_sampling_loc")
    close(ga.cpu().numpy(), ra, BWD_TOL, "grad_attn_weight")


def test_pixel_centres_are_exact(msda):
    """A point at a pixel centre with weight 1 returns the stored row exactly."""
    shapes = ((8, 16), (4, 8))
    w = workloads.random_case(400, 2, shapes, 40, 4, 32, 2)
    rng = np.random.Generator(np.random.PCG64(1))
    loc = w.sampling_loc.copy()
    attn = np.zeros_like(w.attn_weight)
    expect = np.zeros((2, 40, 4, 32), np.float32)
    for b in range(2):
        for q in range(40):
            for m in range(4):
                l = int(rng.integers(2))
                H, W = shapes[l]
                i, j = int(rng.integers(H)), int(rng.integers(W))
                loc[b, q, m, l, 0] = ((j + 0.5) / W, (i + 0.5) / H)
                attn[b, q, m, l, 0] = 1.0
                expect[b, q, m] = w.value[b, w.level_start_index[l] + i * W + j, m]
    w.sampling_loc, w.attn_weight = loc, attn
    _say("pixel centres")
    got = gpu_forward(msda, w).reshape(expect.shape)
    assert np.array_equal(got, expect)


def test_out_of_map_and_nonfinite(msda):
    w = workloads.random_case(500, 2, ((6, 5), (3, 3)), 33, 2, 8, 3)
    loc = w.sampling_loc.copy()
    loc[:, ::2, :, :, :, 0] = -0.5                  # fully left of every map
    loc[:, 1::4, :, :, :, 1] = 1.7                  # fully below
    loc[:, 3, 0, 0, 0, 0] = np.nan
    loc[:, 5, 1, 1, 2, 1] = np.inf
    loc[:, 7, 0, 1, 1, 0] = -np.inf
    w.sampling_loc = loc
    _say("out of map / non-finite")
    got, _ = check_fwd(msda, w)
    assert np.all(np.isfinite(got))
    assert np.all(got.reshape(2, 33, -1)[:, ::2] == 0.0)
    gv, gl, ga = gpu_backward(msda, w)
    rv, rl, ra = oracle_bwd(w)
    assert np.all(np.isfinite(gl)) and np.all(np.isfinite(ga))
    assert np.all(gl[:, ::2] == 0.0) and np.all(ga[:, ::2] == 0.0)
    for x, r in ((gv, rv), (gl, rl), (ga, ra)):
        close(x, r, BWD_TOL)


# ---------------------------------------------------------------------------
# small problems: the one-kernel backward and the binned pipeline
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("D,bf16,acc,align", [(4, False, False, False), (16, False, False, True),
                                              (32, False, True, False), (64, True, False, True),
                                              (128, True, True, False), (256, False, False, False)])
def test_small_backward_both_paths(msda, D, bf16, acc, align):
    """Heads of at most 256 points take the one-kernel backward (workgroups of
    256 pixels: several per head on the 33x40 level); binned=True forces the
    pipeline.  Both against the oracle, with points outside the maps and a
    ragged query count."""
    shapes = ((33, 40), (5, 7), (3, 4)) if D <= 64 else ((4, 5), (2, 3))
    w = workloads.random_case(800 + D, 3, shapes, 19, 3, D, 3, -0.2, 1.2, bf16=bf16)
    _say(f"small backward D={D} bf16={bf16} accumulate={acc} align={align}")
    x = dev_inputs(w, bf16)
    g = torch.from_numpy(w.grad_out).cuda()
    mode = oracle.SPEC | (oracle.ALIGN if align else 0)
    rv, rl, ra = oracle_bwd(w, mode=mode)
    base = torch.randn(tuple(x["value"].shape), generator=torch.Generator().manual_seed(D)).cuda()
    for binned in (False, True):
        gv = base.clone()
        gv, gl, ga = msda.backward(**x, grad_out=g, grad_value=gv, accumulate=acc,
                                   align_corners=align, binned=binned)
        torch.cuda.synchronize()
        dv = gv.cpu().numpy() - (base.cpu().numpy() if acc else 0.0)
        close(dv, rv, BWD_TOL, f"grad_value binned={binned}")
        close(gl.cpu().numpy(), rl, BWD_TOL, f"grad_sampling_loc binned={binned}")
        close(ga.cpu().numpy(), ra, BWD_TOL, f"grad_attn_weight binned={binned}")


# ---------------------------------------------------------------------------
# a seeded sweep of random small problems through every backward path
# ---------------------------------------------------------------------------
def _sweep_case(i):
    """Shape i of the sweep: 1-4 levels of 1..40 x 1..40, Nq 1..150, M 1..6,
    any supported D, K 1..6, fp32 or bf16 value, either pixel convention."""
    rng = np.random.Generator(np.random.PCG64(9000 + i))
    L = int(rng.integers(1, 5))
    shapes = tuple((int(rng.integers(1, 41)), int(rng.integers(1, 41))) for _ in range(L))
    D = int(rng.choice([4, 8, 16, 32, 64, 128, 256]))
    B, Nq, M, K = (int(rng.integers(1, 4)), int(rng.integers(1, 151)), int(rng.integers(1, 7)),
                   int(rng.integers(1, 7)))
    bf16, align = bool(rng.integers(2)), bool(rng.integers(2))
    return shapes, B, Nq, M, D, K, bf16, align


@pytest.mark.parametrize("i", range(48))
def test_random_sweep(msda, i):
    """Forward and both backward paths (the one-kernel path where the heads
    have <= 256 points, the binned pipeline always) against the oracle."""
    shapes, B, Nq, M, D, K, bf16, align = _sweep_case(i)
    _say(f"sweep {i}: shapes={shapes} B={B} Nq={Nq} M={M} D={D} K={K} bf16={bf16} "
         f"align={align}")
    w = workloads.random_case(9100 + i, B, shapes, Nq, M, D, K, -0.15, 1.15, bf16=bf16)
    x = dev_inputs(w, bf16)
    mode = oracle.SPEC | (oracle.ALIGN if align else 0)
    out = msda.forward(**x, align_corners=align)
    g = torch.from_numpy(w.grad_out).cuda()
    torch.cuda.synchronize()
    close(out.cpu().numpy(), oracle_fwd(w, mode=mode).reshape(out.shape), FWD_TOL, "forward")
    rv, rl, ra = oracle_bwd(w, mode=mode)
    for binned in (False, True):
        gv, gl, ga = msda.backward(**x, grad_out=g, align_corners=align, binned=binned)
        torch.cuda.synchronize()
        close(gv.cpu().numpy(), rv, BWD_TOL, f"grad_value binned={binned}")
        close(gl.cpu().numpy(), rl, BWD_TOL, f"grad_sampling_loc binned={binned}")
        close(ga.cpu().numpy(), ra, BWD_TOL, f"grad_attn_weight binned={binned}")


def test_empty_inputs(msda):
    d = torch.device("cuda:0")
    _say("empty")
    ss = torch.tensor([[4, 4]], device=d)
    st = torch.tensor([0], device=d)
    # no queries
    v = torch.randn(2, 16, 2, 8, device=d)
    loc = torch.zeros(2, 0, 2, 1, 3, 2, device=d)
    a = torch.zeros(2, 0, 2, 1, 3, device=d)
    out = msda.forward(v, ss, st, loc, a)
    assert out.shape == (2, 0, 16)
    gv, gl, ga = msda.backward(v, ss, st, loc, a, torch.zeros(2, 0, 16, device=d))
    torch.cuda.synchronize()
    assert torch.count_nonzero(gv).item() == 0          # overwritten with zeros
    # no batch
    v = torch.randn(0, 16, 2, 8, device=d)
    out = msda.forward(v, ss, st, torch.zeros(0, 5, 2, 1, 3, 2, device=d),
                       torch.zeros(0, 5, 2, 1, 3, device=d))
    assert out.shape == (0, 5, 16)


def test_accumulate_adds_into_grad_value(msda):
    w = workloads.random_case(600, 2, ((7, 9), (3, 4)), 50, 2, 32, 4)
    x = dev_inputs(w)
    g = torch.from_numpy(w.grad_out).cuda()
    base = torch.randn(x["value"].shape, device="cuda")
    gv = base.clone()
    _say("accumulate")
    msda.backward(**x, grad_out=g, grad_value=gv, accumulate=True)
    torch.cuda.synchronize()
    rv, _, _ = oracle_bwd(w)
    close(gv.cpu().numpy() - base.cpu().numpy(), rv, BWD_TOL)


@pytest.mark.parametrize("D", [8, 32, 64])
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("acc", [False, True])
def test_split_bins(msda, D, bf16, acc):
    # a 5x6 level is one 8x8 tile: 1500 queries x 4 points per head put ~6000
    # records in its bin, which the work list splits into three items; their
    # partial tiles are added up by the combine kernel (D <= 32) or atomically
    # into the zeroed tile (D = 64), onto earlier contents with acc
    w = workloads.random_case(1900 + D, 2, ((5, 6), (12, 10)), 1500, 2, D, 4, bf16=bf16)
    x = dev_inputs(w, bf16)
    g = torch.from_numpy(w.grad_out).cuda()
    base = torch.randn(w.value.shape, device="cuda") if acc else None
    _say(f"split bins D={D} bf16={bf16} acc={acc}")
    # overwrite mode starts from NaN: every element must be written
    gv0 = base.clone() if acc else torch.full(tuple(w.value.shape), float("nan"), device="cuda")
    gv, gl, ga = msda.backward(**x, grad_out=g, grad_value=gv0, accumulate=acc)
    torch.cuda.synchronize()
    rv, rl, ra = oracle_bwd(w)
    got_v = gv.cpu().numpy() - (base.cpu().numpy() if acc else 0.0)
    close(got_v, rv, BWD_TOL, "grad_value")
    close(gl.cpu().numpy(), rl, BWD_TOL, "grad_sampling_loc")
    close(ga.cpu().numpy(), ra, BWD_TOL, "grad_attn_weight")


@pytest.mark.parametrize("acc", [False, True])
def test_split_bins_many_items(msda, acc):
    # one level of one tile: 6000 queries x 4 points per head, 24000 points
    # and up to four records each in one bin, split into a dozen or more
    # items of unequal, balanced sizes
    w = workloads.random_case(1950, 1, ((5, 6),), 6000, 2, 32, 4)
    x = dev_inputs(w)
    g = torch.from_numpy(w.grad_out).cuda()
    base = torch.randn(w.value.shape, device="cuda") if acc else None
    _say(f"split bins, many items, acc={acc}")
    # overwrite mode starts from NaN: every element must be written
    gv0 = base.clone() if acc else torch.full(tuple(w.value.shape), float("nan"), device="cuda")
    gv, gl, ga = msda.backward(**x, grad_out=g, grad_value=gv0, accumulate=acc)
    torch.cuda.synchronize()
    rv, rl, ra = oracle_bwd(w)
    got_v = gv.cpu().numpy() - (base.cpu().numpy() if acc else 0.0)
    close(got_v, rv, BWD_TOL, "grad_value")
    close(gl.cpu().numpy(), rl, BWD_TOL, "grad_sampling_loc")
    close(ga.cpu().numpy(), ra, BWD_TOL, "grad_attn_weight")


@pytest.mark.parametrize("D", [32, 64])
@pytest.mark.parametrize("acc", [False, True])
def test_scan_two_passes(msda, D, acc):
    # 2 batches x 8 heads x (256 + 1) tiles = 4112 bins: the scan takes two
    # passes of 4096, and both hold empty bins (the points crowd into a corner
    # of the 128x128 level) and split bins (the 5x6 level is one tile with
    # ~6000 records per head); overwrite mode starts from NaN
    w = workloads.random_case(1970 + D, 2, ((128, 128), (5, 6)), 1500, 8, D, 4, 0.0, 0.3)
    x = dev_inputs(w)
    g = torch.from_numpy(w.grad_out).cuda()
    base = torch.randn(w.value.shape, device="cuda") if acc else None
    _say(f"two-pass scan D={D} acc={acc}")
    gv0 = base.clone() if acc else torch.full(tuple(w.value.shape), float("nan"), device="cuda")
    gv, gl, ga = msda.backward(**x, grad_out=g, grad_value=gv0, accumulate=acc)
    torch.cuda.synchronize()
    rv, rl, ra = oracle_bwd(w)
    got_v = gv.cpu().numpy() - (base.cpu().numpy() if acc else 0.0)
    assert np.all(np.isfinite(got_v))
    close(got_v, rv, BWD_TOL, "grad_value")
    close(gl.cpu().numpy(), rl, BWD_TOL, "grad_sampling_loc")
    close(ga.cpu().numpy(), ra, BWD_TOL, "grad_attn_weight")


@pytest.mark.parametrize("D,acc", [(8, False), (8, True), (64, False)])
def test_scan_many_blocks(msda, D, acc):
    """8 batches x 8 heads x (320 + 80 + 20) tiles = 26,880 bins: seven scan
    workgroups, each summing the counts of the blocks before its own; few
    points (200 queries), so most bins are empty and, with the gather kernel
    (D = 8), the zero list runs through every block (D = 64 takes the tile
    kernel, and such a sparse problem has grad_value zero-filled whole).
    Overwrite mode starts from NaN."""
    w = workloads.random_case(1980 + D, 8, ((128, 160), (64, 80), (32, 40)), 200, 8, D, 2)
    x = dev_inputs(w)
    g = torch.from_numpy(w.grad_out).cuda()
    base = torch.randn(w.value.shape, device="cuda") if acc else None
    _say(f"many-block scan D={D} acc={acc}")
    gv0 = base.clone() if acc else torch.full(tuple(w.value.shape), float("nan"), device="cuda")
    gv, gl, ga = msda.backward(**x, grad_out=g, grad_value=gv0, accumulate=acc, binned=True)
    torch.cuda.synchronize()
    rv, rl, ra = oracle_bwd(w)
    got_v = gv.cpu().numpy() - (base.cpu().numpy() if acc else 0.0)
    assert np.all(np.isfinite(got_v))
    close(got_v, rv, BWD_TOL, "grad_value")
    close(gl.cpu().numpy(), rl, BWD_TOL, "grad_sampling_loc")
    close(ga.cpu().numpy(), ra, BWD_TOL, "grad_attn_weight")


def test_runs_on_the_callers_stream(msda):
    w = workloads.random_case(700, 2, ((9, 9), (4, 4)), 90, 4, 32, 4)
    x = dev_inputs(w)
    s = torch.cuda.Stream()
    _say("side stream")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out = msda.forward(**x, validate=False)
        gv, gl, ga = msda.backward(**x, grad_out=torch.from_numpy(w.grad_out).cuda(),
                                   validate=False)
        # consumers enqueued on the same stream, with no host synchronization:
        # they must see every output complete (the backward joins its side
        # stream back into the caller's stream)
        gv2, gl2, ga2 = gv.clone(), gl.clone(), ga.clone()
    s.synchronize()
    close(out.cpu().numpy(), oracle_fwd(w), FWD_TOL)
    rv, rl, ra = oracle_bwd(w)
    close(gv2.cpu().numpy(), rv, BWD_TOL, "grad_value")
    close(gl2.cpu().numpy(), rl, BWD_TOL, "grad_sampling_loc")
    close(ga2.cpu().numpy(), ra, BWD_TOL, "grad_attn_weight")


def test_autograd_function(msda):
    w = workloads.random_case(800, 1, ((6, 7), (3, 3)), 20, 2, 16, 2)
    x = dev_inputs(w)
    v = x["value"].clone().requires_grad_(True)
    loc = x["sampling_loc"].clone().requires_grad_(True)
    a = x["attn_weight"].clone().requires_grad_(True)
    _say("autograd")
    out = msda.ms_deform_attn(v, x["spatial_shapes"], x["level_start_index"], loc, a)
    out.backward(torch.from_numpy(w.grad_out).cuda())
    rv, rl, ra = oracle_bwd(w)
    close(out.detach().cpu().numpy(), oracle_fwd(w), FWD_TOL)
    close(v.grad.cpu().numpy(), rv, BWD_TOL)
    close(loc.grad.cpu().numpy(), rl, BWD_TOL)
    close(a.grad.cpu().numpy(), ra, BWD_TOL)


def test_backward_repeatability(msda):
    """grad_value is summed with atomics in no fixed order: report the spread
    over repeated runs; grad_loc and grad_attn are deterministic."""
    w = workloads.make(3)
    x = dev_inputs(w)
    g = torch.from_numpy(w.grad_out).cuda()
    _say("repeatability x5 encoder bwd")
    runs = [tuple(t.clone() for t in msda.backward(**x, grad_out=g, validate=False))
            for _ in range(5)]
    torch.cuda.synchronize()
    ref = runs[0]
    scale = ref[0].abs().max().item()
    spread = max((r[0] - ref[0]).abs().max().item() for r in runs[1:]) / scale
    print(f"grad_value spread over 5 runs: {spread:.3e} (relative to max)", flush=True)
    assert spread <= 1e-5
    for r in runs[1:]:
        assert torch.equal(r[1], ref[1]) and torch.equal(r[2], ref[2])


@pytest.mark.parametrize("accumulate", [False, True])
def test_backward_with_stage_events(msda, accumulate):
    """msda_backward_events gives the same gradients as the oracle and records a
    start and an end event around every stage."""
    w = workloads.random_case(900, 2, ((9, 13), (5, 7)), 70, 4, 32, 4)
    x = dev_inputs(w)
    g = torch.from_numpy(w.grad_out).cuda()
    _say(f"backward with stage events, accumulate={accumulate}")
    ev = msda.make_events()
    gv0 = torch.zeros(x["value"].shape, device="cuda") if accumulate else None
    gv, gl, ga = msda.backward(**x, grad_out=g, grad_value=gv0, accumulate=accumulate, events=ev)
    torch.cuda.synchronize()
    st = msda.stage_times(ev)
    assert len(st) == len(msda.BWD_STAGES) and all(t >= 0.0 for t in st)
    assert st[msda.BWD_STAGES.index("tiles")] > 0.0 and st[msda.BWD_STAGES.index("dots")] > 0.0
    rv, rl, ra = oracle_bwd(w)
    close(gv.cpu().numpy(), rv, BWD_TOL, "grad_value")
    close(gl.cpu().numpy(), rl, BWD_TOL, "grad_sampling_loc")
    close(ga.cpu().numpy(), ra, BWD_TOL, "grad_attn_weight")


@pytest.mark.parametrize("side", ["auto", None])
def test_stage_events_span_passes(msda, side):
    """With grad_value in passes (the smallest workspace: 1024-query ranges of
    one head), each stage's events run from its start in the first pass to
    its end in the last: every stage is timed, and the gradients match the
    oracle."""
    w = workloads.random_case(910, 2, ((40, 56), (20, 28)), 2300, 2, 32, 4)
    B, Nv, Nq, M, D, L, K = (w.dims[k] for k in ("B", "Nv", "Nq", "M", "D", "L", "K"))
    least = msda.workspace_min(B, Nv, Nq, M, D, L, K)
    x = dev_inputs(w)
    g = torch.from_numpy(w.grad_out).cuda()
    _say(f"stage events over passes, side_stream={side}")
    ev = msda.make_events()
    gv, gl, ga = msda.backward(**x, grad_out=g, events=ev, side_stream=side,
                               workspace=torch.empty(least, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    st = msda.stage_times(ev)
    assert len(st) == len(msda.BWD_STAGES) and all(t >= 0.0 for t in st)
    assert st[msda.BWD_STAGES.index("tiles")] > 0.0 and st[msda.BWD_STAGES.index("count")] > 0.0
    rv, rl, ra = oracle_bwd(w)
    close(gv.cpu().numpy(), rv, BWD_TOL, "grad_value")
    close(gl.cpu().numpy(), rl, BWD_TOL, "grad_sampling_loc")
    close(ga.cpu().numpy(), ra, BWD_TOL, "grad_attn_weight")


def test_two_streams_backward_concurrently(msda):
    """Two backwards issued on two torch streams without a host wait between
    them, each with its own workspace (and, by default, its own side stream
    kept by the binding), compared with the oracle: the library holds no state
    that the two calls share."""
    wa = workloads.random_case(1200, 2, ((40, 52), (20, 26), (10, 13)), 900, 4, 32, 4)
    wb = workloads.random_case(1201, 1, ((33, 17), (9, 9)), 1300, 8, 16, 3, -0.2, 1.2)
    xa, xb = dev_inputs(wa), dev_inputs(wb)
    ga, gb = torch.from_numpy(wa.grad_out).cuda(), torch.from_numpy(wb.grad_out).cuda()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    _say("two streams, concurrent backwards")
    with torch.cuda.stream(sa):
        ra = msda.backward(**xa, grad_out=ga, validate=False)
    with torch.cuda.stream(sb):
        rb = msda.backward(**xb, grad_out=gb, validate=False)
    torch.cuda.synchronize()
    for got, w in ((ra, wa), (rb, wb)):
        for x, r, n in zip(got, oracle_bwd(w), ("grad_value", "grad_sampling_loc",
                                                "grad_attn_weight")):
            close(x.cpu().numpy(), r, BWD_TOL, f"{w.name} {n}")


@pytest.mark.parametrize("side", ["auto", None])
@pytest.mark.parametrize("acc", [False, True])
@pytest.mark.parametrize("budget", ["min", "heads", "batches", "queries"])
def test_backward_in_passes(msda, budget, acc, side):
    """A workspace below workspace_size: grad_value in passes, each a box of
    batches x heads x queries run as a problem of its own, the passes after
    a query range's first adding to grad_value.  Budgets (3 batches, 4 heads,
    2500 queries): "batches" holds 2 whole batches (passes of 2 and 1);
    "queries" 1500 queries of every head of one batch (6 passes: 1500 +
    1000 a batch); "heads" 1024 queries of two heads (18 passes); "min"
    (workspace_min) 1024 queries of one head (36 passes: 1024 + 1024 + 452).
    Overwrite mode starts from NaN.  On one stream (side None) the dots kernel
    clears the first pass's bin counters and the later passes clear their own."""
    w = workloads.random_case(1500, 3, ((40, 56), (20, 28), (10, 14), (5, 7)), 2500, 4, 32, 4)
    B, Nv, Nq, M, D, L, K = (w.dims[k] for k in ("B", "Nv", "Nq", "M", "D", "L", "K"))
    full = msda.workspace_size(B, Nv, Nq, M, D, L, K)
    nbytes = {"min": msda.workspace_min(B, Nv, Nq, M, D, L, K),
              "heads": msda.workspace_size(1, Nv, 1024, 2, D, L, K),
              "batches": msda.workspace_size(2, Nv, Nq, M, D, L, K),
              "queries": msda.workspace_size(1, Nv, 1500, M, D, L, K)}[budget]
    assert nbytes < full
    _say(f"backward in passes: budget {budget} ({nbytes} of {full} bytes), acc={acc}, "
         f"side_stream={side}")
    x = dev_inputs(w)
    g = torch.from_numpy(w.grad_out).cuda()
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    base = torch.randn(w.value.shape, device="cuda") if acc else None
    gv0 = base.clone() if acc else torch.full(tuple(w.value.shape), float("nan"), device="cuda")
    gv, gl, ga = msda.backward(**x, grad_out=g, grad_value=gv0, accumulate=acc, workspace=ws,
                               side_stream=side)
    torch.cuda.synchronize()
    rv, rl, ra = oracle_bwd(w)
    got_v = gv.cpu().numpy() - (base.cpu().numpy() if acc else 0.0)
    close(got_v, rv, BWD_TOL, "grad_value")
    close(gl.cpu().numpy(), rl, BWD_TOL, "grad_sampling_loc")
    close(ga.cpu().numpy(), ra, BWD_TOL, "grad_attn_weight")


@pytest.mark.parametrize("seed", range(8))
def test_backward_in_passes_random_budgets(msda, seed):
    """Random shapes and workspaces anywhere between workspace_min and
    workspace_size (every plan shape, ragged boxes, both grad_value kernels),
    overwrite from NaN or accumulate, against the oracle."""
    r = np.random.default_rng(1600 + seed)
    B, M = int(r.integers(1, 4)), int(r.integers(1, 5))
    Nq, K = int(r.integers(300, 2600)), int(r.integers(1, 5))
    D = int(r.choice([8, 16, 32, 64, 128]))
    L = int(r.integers(1, 4))
    shapes = tuple((int(r.integers(3, 40)), int(r.integers(3, 60))) for _ in range(L))
    acc = bool(r.integers(0, 2))
    w = workloads.random_case(1610 + seed, B, shapes, Nq, M, D, K)
    Nv = w.dims["Nv"]
    lo, hi = msda.workspace_min(B, Nv, Nq, M, D, L, K), msda.workspace_size(B, Nv, Nq, M, D, L, K)
    nbytes = int(r.integers(lo, hi)) if hi > lo else lo
    _say(f"passes, random budget: B={B} M={M} Nq={Nq} D={D} L={L} K={K} shapes={shapes} "
         f"acc={acc} workspace {nbytes} of [{lo}, {hi}]")
    x = dev_inputs(w)
    g = torch.from_numpy(w.grad_out).cuda()
    base = torch.randn(w.value.shape, device="cuda") if acc else None
    gv0 = base.clone() if acc else torch.full(tuple(w.value.shape), float("nan"), device="cuda")
    gv, gl, ga = msda.backward(**x, grad_out=g, grad_value=gv0, accumulate=acc,
                               workspace=torch.empty(nbytes, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    rv, rl, ra = oracle_bwd(w)
    got_v = gv.cpu().numpy() - (base.cpu().numpy() if acc else 0.0)
    close(got_v, rv, BWD_TOL, "grad_value")
    close(gl.cpu().numpy(), rl, BWD_TOL, "grad_sampling_loc")
    close(ga.cpu().numpy(), ra, BWD_TOL, "grad_attn_weight")


def test_backward_in_passes_bf16_align_corners(msda):
    """Query-range passes (room for 1100 queries of every head: 2 passes a
    batch) with a bf16 value and the align_corners convention, against the
    oracle on the bf16-rounded value in that convention."""
    w = workloads.random_case(1520, 2, ((40, 56), (20, 28), (10, 14)), 2200, 4, 32, 4,
                              -0.1, 1.1, bf16=True)
    B, Nv, Nq, M, D, L, K = (w.dims[k] for k in ("B", "Nv", "Nq", "M", "D", "L", "K"))
    nbytes = msda.workspace_size(1, Nv, 1100, M, D, L, K)
    _say(f"backward in passes, bf16 value, align_corners ({nbytes} bytes)")
    x = dev_inputs(w, bf16=True)
    g = torch.from_numpy(w.grad_out).cuda()
    gv, gl, ga = msda.backward(**x, grad_out=g, align_corners=True,
                               workspace=torch.empty(nbytes, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    rv, rl, ra = oracle_bwd(w, mode=oracle.SPEC | oracle.ALIGN)
    close(gv.cpu().numpy(), rv, BWD_TOL, "grad_value")
    close(gl.cpu().numpy(), rl, BWD_TOL, "grad_sampling_loc")
    close(ga.cpu().numpy(), ra, BWD_TOL, "grad_attn_weight")


@pytest.mark.parametrize("D", [16, 128])
def test_backward_head_passes_tile_kernel_and_sparse(msda, D):
    """Head passes through both grad_value kernels: D = 128 takes the tile
    kernel (the 5x6 level's one tile, 2400 records a head, split and added
    atomically into its zeroed tile); the sparse maps (few points per pixel,
    otherwise zero-filled whole) have most tiles empty, zeroed from the list."""
    w = workloads.random_case(1510 + D, 2, ((64, 96), (32, 48), (5, 6)), 600, 3, D, 4)
    B, Nv, Nq, M, _, L, K = (w.dims[k] for k in ("B", "Nv", "Nq", "M", "D", "L", "K"))
    # room for two of the three heads of 600 queries: passes of heads {0, 1}
    # and {2} of each batch
    nbytes = msda.workspace_size(1, Nv, Nq, 2, D, L, K)
    _say(f"head passes D={D} ({nbytes} bytes)")
    x = dev_inputs(w)
    g = torch.from_numpy(w.grad_out).cuda()
    gv0 = torch.full(tuple(w.value.shape), float("nan"), device="cuda")
    gv, gl, ga = msda.backward(**x, grad_out=g, grad_value=gv0,
                               workspace=torch.empty(nbytes, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    rv, rl, ra = oracle_bwd(w)
    close(gv.cpu().numpy(), rv, BWD_TOL, "grad_value")
    close(gl.cpu().numpy(), rl, BWD_TOL, "grad_sampling_loc")
    close(ga.cpu().numpy(), ra, BWD_TOL, "grad_attn_weight")


def test_one_stream_matches_side_stream_at_encoder_shape(msda):
    """The encoder shape on one stream (the dots kernel then also clears the
    bin counters) against the side-stream run: the point gradients are
    deterministic and equal bit for bit, grad_value equal to summation order."""
    w = workloads.make(3)
    x = dev_inputs(w)
    g = torch.from_numpy(w.grad_out).cuda()
    _say("encoder backward, one stream against side stream")
    a = msda.backward(**x, grad_out=g, validate=False, side_stream="auto")
    b = msda.backward(**x, grad_out=g, validate=False, side_stream=None)
    torch.cuda.synchronize()
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    close(b[0].cpu().numpy(), a[0].cpu().numpy(), 1e-5, "grad_value")


def test_backward_below_min_workspace_raises(msda):
    w = workloads.random_case(1501, 1, ((40, 56), (20, 28)), 2000, 2, 16, 4)
    B, Nv, Nq, M, D, L, K = (w.dims[k] for k in ("B", "Nv", "Nq", "M", "D", "L", "K"))
    least = msda.workspace_min(B, Nv, Nq, M, D, L, K)
    x = dev_inputs(w)
    g = torch.from_numpy(w.grad_out).cuda()
    with pytest.raises(ValueError):
        msda.backward(**x, grad_out=g, workspace=torch.empty(least - 256, dtype=torch.uint8,
                                                              device="cuda"))


@pytest.mark.parametrize("side", ["auto", None])
def test_overwrite_replaces_every_element(msda, side):
    """Overwrite mode writes every element of grad_value: a NaN-filled buffer
    comes back equal to the oracle.  The points crowd into a corner of each
    map, so most 8x8 tiles receive nothing (zeroed from the zero list), and
    the small coarse level's one tile is split over several work items.
    288,000 points: enough for the backward to use the side stream."""
    w = workloads.random_case(1300, 2, ((48, 64), (24, 32), (5, 6)), 1500, 8, 32, 4,
                              0.0, 0.3)
    x = dev_inputs(w)
    g = torch.from_numpy(w.grad_out).cuda()
    _say(f"overwrite of a NaN-filled grad_value, side_stream={side}")
    gv = torch.full(tuple(w.value.shape), float("nan"), device="cuda")
    gv, gl, ga = msda.backward(**x, grad_out=g, grad_value=gv, side_stream=side)
    torch.cuda.synchronize()
    rv, rl, ra = oracle_bwd(w)
    got = gv.cpu().numpy()
    assert np.all(np.isfinite(got))
    close(got, rv, BWD_TOL, "grad_value")
    close(gl.cpu().numpy(), rl, BWD_TOL, "grad_sampling_loc")
    close(ga.cpu().numpy(), ra, BWD_TOL, "grad_attn_weight")
