"""GPU parity of DAT's sampled-key attention: the sampling step (msda_forward
/ msda_backward with one level, one point, weight 1, align_corners) and the
MFMA attention (msda_dat_attention_forward / _backward) against the CPU
oracle (oracle/dat.py).  Metric max|x - r| / max|r|: forward 1e-5, backward
1e-4 (dK, dV may be summed with atomics over query ranges)."""
import numpy as np
import pytest
import torch

import oracle
import oracle.dat as odat
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


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def check_attention(m, w, with_grad_bias=True, scale=None):
    q, k, v = _t(w.q), _t(w.k), _t(w.v)
    bias = _t(w.bias) if w.bias is not None else None
    out, lse = m.dat_attention(q, k, v, bias, scale)
    torch.cuda.synchronize()
    r_out, r_lse = odat.attention(w.q, w.k, w.v, w.bias, scale)
    e = max_rel(out.cpu().numpy(), r_out)
    assert e <= FWD_TOL, f"{w.name}: attention out max rel {e:.3e}"
    e = max_rel(lse.cpu().numpy(), r_lse)
    assert e <= FWD_TOL, f"{w.name}: lse max rel {e:.3e}"
    g = _t(w.grad_out)
    gq, gk, gv, gb = m.dat_attention_backward(q, k, v, out, lse, g, bias,
                                              need_grad_bias=with_grad_bias, scale=scale)
    torch.cuda.synchronize()
    rq, rk, rv, rb = odat.attention_backward(w.q, w.k, w.v, w.grad_out, w.bias, scale)
    got = [("dq", gq, rq), ("dk", gk, rk), ("dv", gv, rv)]
    if w.bias is not None and with_grad_bias:
        got.append(("dbias", gb, rb))
    for name, a, r in got:
        e = max_rel(a.cpu().numpy(), r)
        assert e <= BWD_TOL, f"{w.name}: {name} max rel {e:.3e}"


@pytest.mark.parametrize("heads,C", [(2, 32), (3, 96), (1, 64)])   # head dims 16, 32, 64
@pytest.mark.parametrize("hw,khw", [((5, 7), (1, 1)), ((9, 11), (3, 4)), ((14, 14), (7, 7)),
                                    ((16, 20), (10, 10))])
def test_dat_attention_shapes(msda, heads, C, hw, khw):
    _say(f"dat attention heads={heads} C={C} N={hw} Ns={khw}")
    w = workloads.dat_case(3000 + heads + C + hw[0] + khw[0], 2, hw[0], hw[1], C, heads, 1,
                           khw[0], khw[1])
    check_attention(msda, w)


def test_dat_attention_no_bias_and_scale(msda):
    _say("dat attention without bias, explicit scale")
    w = workloads.dat_case(3101, 3, 12, 10, 64, 2, 1, 5, 4, with_bias=False)
    check_attention(msda, w, scale=0.37)


def test_dat_attention_query_splits(msda):
    # few (batch, head) pairs and many queries: the dK/dV kernel splits the
    # queries over several workgroups and adds with atomics
    _say("dat attention query splits")
    w = workloads.dat_case(3201, 1, 20, 25, 64, 2, 1, 6, 7)
    check_attention(msda, w)


def test_dat_attention_large_scores(msda):
    # scores of tens: the softmax must subtract its maximum
    _say("dat attention large scores")
    w = workloads.dat_case(3301, 2, 8, 8, 64, 2, 1, 4, 4)
    check_attention(msda, w, scale=4.0)


def test_dat_attention_max_keys(msda):
    _say("dat attention Ns=256, head_dim 32")
    w = workloads.dat_case(3401, 1, 9, 9, 64, 2, 1, 16, 16)
    check_attention(msda, w)


# key counts that select each kernel build (key blocks 2, 8, 16) and LDS mode:
# K and V resident together, or one buffer (head_dim 64 with >= 113 keys,
# head_dim 32 with > 240); Ns % 4 != 0 reads the bias rows unaligned
@pytest.mark.parametrize("heads,C,khw", [(2, 64, (5, 5)), (1, 64, (16, 15)), (2, 128, (8, 16)),
                                         (2, 128, (7, 17)), (1, 16, (16, 16))])
def test_dat_attention_key_blocks(msda, heads, C, khw):
    _say(f"dat attention key blocks heads={heads} C={C} Ns={khw}")
    w = workloads.dat_case(3701 + C + khw[0] * khw[1], 2, 7, 9, C, heads, 1, khw[0], khw[1])
    check_attention(msda, w)


def test_dat_attention_query_tiles(msda):
    # 8 * 16 (batch, head) pairs of 1000 queries: enough workgroups that each
    # wave takes two 16-query tiles, the last workgroup of each pair ragged
    _say("dat attention several query tiles per wave")
    w = workloads.dat_case(3801, 8, 25, 40, 256, 16, 1, 3, 5)
    check_attention(msda, w)


@pytest.mark.parametrize("C,heads,khw,hw", [(64, 4, (7, 7), (7, 9)), (128, 4, (8, 8), (5, 13)),
                                             (256, 4, (7, 8), (4, 4))])
def test_dat_attention_one_kernel_backward(msda, C, heads, khw, hw):
    # 49..64 keys and >= 256 (batch, head) pairs: the one-kernel backward
    # (head widths 16, 32, 64; ragged query tiles; bias and its gradient)
    _say(f"dat attention one-kernel backward C={C} heads={heads} Ns={khw} N={hw}")
    w = workloads.dat_case(3901 + C, 64, hw[0], hw[1], C, heads, 1, khw[0], khw[1])
    check_attention(msda, w)


@pytest.mark.parametrize("i", range(24))
def test_dat_attention_sweep(msda, i):
    # seeded random shapes across the kernels' builds: 1..256 keys, head
    # widths 16/32/64 (keys <= 240 at 64), 1..600 queries, 1..48 (b, head)
    # pairs, with or without the bias
    rng = np.random.Generator(np.random.PCG64(9500 + i))
    d = int(rng.choice([16, 32, 64]))
    hk, wk = int(rng.integers(1, 17)), int(rng.integers(1, 17))
    while hk * wk > (240 if d == 64 else 256):
        hk -= 1
    H, W = int(rng.integers(1, 25)), int(rng.integers(1, 26))
    heads, B = int(rng.integers(1, 5)), int(rng.integers(1, 13))
    with_bias = bool(rng.integers(2))
    _say(f"dat attention sweep {i}: B={B} N={H * W} Ns={hk * wk} heads={heads} d={d} "
         f"bias={with_bias}")
    w = workloads.dat_case(9600 + i, B, H, W, heads * d, heads, 1, hk, wk, with_bias=with_bias)
    check_attention(msda, w)


def test_dat_attention_empty(msda):
    _say("dat attention N=0")
    k = torch.randn(2, 5, 2, 32, device="cuda")
    v = torch.randn(2, 5, 2, 32, device="cuda")
    q = torch.zeros(2, 0, 2, 32, device="cuda")
    out, lse = msda.dat_attention(q, k, v)
    gq, gk, gv, _ = msda.dat_attention_backward(q, k, v, out, lse, torch.zeros_like(q))
    torch.cuda.synchronize()
    assert out.shape == (2, 0, 2, 32) and float(gk.abs().max()) == 0.0
    assert float(gv.abs().max()) == 0.0


@pytest.mark.parametrize("G", [1, 3])
def test_dat_sampling(msda, G):
    _say(f"dat sampling G={G}")
    # 32 channels per group (the core takes power-of-two head widths)
    w = workloads.dat_case(3501 + G, 2, 13, 17, 32 * G, G, G, 5, 6, offset_cells=1.5)
    x, pos = _t(w.x), _t(w.pos)
    smp = msda.dat_sample(x, w.hw, pos)
    gx, gp = msda.dat_sample_backward(x, w.hw, pos, _t(w.grad_sampled))
    torch.cuda.synchronize()
    assert max_rel(smp.cpu().numpy(), odat.sample(w.x, w.hw, w.pos)) <= FWD_TOL
    rx, rp = odat.sample_backward(w.x, w.hw, w.pos, w.grad_sampled)
    assert max_rel(gx.cpu().numpy(), rx) <= BWD_TOL
    assert max_rel(gp.cpu().numpy(), rp) <= BWD_TOL


def test_dat_autograd(msda):
    _say("dat autograd: sampling -> attention")
    w = workloads.dat_case(3601, 2, 10, 12, 64, 2, 2, 4, 5)
    x = _t(w.x).requires_grad_(True)
    pos = _t(w.pos).requires_grad_(True)
    q = _t(w.q).requires_grad_(True)
    bias = _t(w.bias).requires_grad_(True)
    smp = msda.DATSampleFunction.apply(x, w.hw, pos)             # [B, Ns, C]
    B, Ns, C = smp.shape
    kv = smp.reshape(B, Ns, 2, C // 2)                            # identity projections
    out = msda.dat_deformable_attention(q, kv, kv, bias)
    out.backward(_t(w.grad_out))
    torch.cuda.synchronize()
    # oracle: the same composition
    s = odat.sample(w.x, w.hw, w.pos).reshape(B, Ns, 2, C // 2)
    r_out, _ = odat.attention(w.q, s, s, w.bias)
    assert max_rel(out.detach().cpu().numpy(), r_out) <= FWD_TOL
    dq, dk, dv, db = odat.attention_backward(w.q, s, s, w.grad_out, w.bias)
    gs = (dk + dv).reshape(B, Ns, C)
    rx, rp = odat.sample_backward(w.x, w.hw, w.pos, gs)
    for name, a, r in (("q", q.grad, dq), ("bias", bias.grad, db), ("x", x.grad, rx),
                       ("pos", pos.grad, rp)):
        assert max_rel(a.cpu().numpy(), r) <= BWD_TOL, name


@pytest.mark.parametrize("name", ["dat_cls", "dat_det"])
def test_dat_configs(msda, name):
    # DAT-T stage 3 at 224 (B=64, 196 tokens, 49 keys) and at 1024 for
    # detection (B=2, 4096 tokens, 256 keys); 12 heads of 32, with a bias
    _say(f"dat config {name}")
    check_attention(msda, workloads.make_dat(name, with_bias=True))
