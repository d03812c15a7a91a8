"""The DAT oracle against its pins, and planted mistakes in copies of it (CPU
only; oracle/dat.py itself is never modified)."""
import importlib.util
import os

import pytest

import oracle
import oracle.dat
from dat_pins import ALL_DAT_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "dat.py")


@pytest.mark.parametrize("pin", ALL_DAT_PINS, ids=[p.__name__ for p in ALL_DAT_PINS])
def test_dat_oracle_pin(pin):
    pin(oracle.dat)


MUTANTS = [
    ("no_scale", "s = scale * np.einsum(\"bnhd,bshd->bhns\", q, k)", "s = np.einsum(\"bnhd,bshd->bhns\", q, k)", 1),
    ("bias_dropped", "s = s + np.asarray(bias, dtype=np.float64)", "s = s", 1),
    ("softmax_over_queries", "mx = s.max(axis=-1, keepdims=True)\n    e = np.exp(s - mx)\n    tot = e.sum(axis=-1, keepdims=True)", "mx = s.max(axis=-1, keepdims=True)\n    e = np.exp(s - mx)\n    tot = e.sum(axis=-2, keepdims=True)", 1),
    ("out_uses_scores", "out = np.einsum(\"bhns,bshd->bnhd\", p, v)", "out = np.einsum(\"bhns,bshd->bnhd\", e, v)", 1),
    ("lse_without_max", "lse = (mx + np.log(tot))[..., 0]", "lse = np.log(tot)[..., 0]", 1),
    ("grad_no_centering", "ds = p * (dp - (p * dp).sum(axis=-1, keepdims=True))", "ds = p * dp", 1),
    ("grad_q_no_scale", "dq = scale * np.einsum(\"bhns,bshd->bnhd\", ds, k)", "dq = np.einsum(\"bhns,bshd->bnhd\", ds, k)", 1),
    ("grad_k_uses_p", "dk = scale * np.einsum(\"bhns,bnhd->bshd\", ds, q)", "dk = scale * np.einsum(\"bhns,bnhd->bshd\", p, q)", 1),
    ("grad_v_uses_ds", "dv = np.einsum(\"bhns,bnhd->bshd\", p, g)", "dv = np.einsum(\"bhns,bnhd->bshd\", ds, g)", 1),
    ("dp_uses_q", "dp = np.einsum(\"bnhd,bshd->bhns\", g, v)", "dp = np.einsum(\"bnhd,bshd->bhns\", g, k)", 1),
    ("sampling_half_pixel", "mode=mode | _core.ALIGN)\n\n\ndef sample_backward", "mode=mode)\n\n\ndef sample_backward", 1),
]


def _load(path, name):
    spec = importlib.util.spec_from_file_location(f"dat_mutant_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,orig,planted,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_dat_mutant_is_caught(tmp_path, name, orig, planted, count):
    src = open(SRC).read()
    assert src.count(orig) == count, f"mutation site for {name} not found"
    path = tmp_path / f"dat_{name}.py"
    path.write_text(src.replace(orig, planted))
    mod = _load(str(path), name)
    caught = None
    for pin in ALL_DAT_PINS:
        try:
            pin(mod)
        except Exception:
            caught = pin.__name__
            break
    assert caught is not None, f"no pin caught the planted mistake {name}"
