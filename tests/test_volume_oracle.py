"""The 3-D (trilinear) oracle against its pins, and planted mistakes in copies
of it (CPU only; oracle/msda3d_oracle.c itself is never modified)."""
import os
import subprocess
import sys

import pytest

import oracle.volume as ov
from volume_pins import ALL_VOLUME_PINS


@pytest.mark.parametrize("pin", ALL_VOLUME_PINS, ids=[p.__name__ for p in ALL_VOLUME_PINS])
def test_volume_oracle_pin(pin):
    pin(ov.default())


# (name, original text, planted text, count)
MUTANTS = [
    ("axes_w_h_swapped", "const int64_t n[3] = {W, H, Z};", "const int64_t n[3] = {H, W, Z};", 1),
    ("z_stride_uses_w", "((int64_t)idx[2] * H + (int64_t)idx[1]) * W", "((int64_t)idx[2] * W + (int64_t)idx[1]) * W", 1),
    ("z_ignored_in_index", "((int64_t)idx[2] * H + (int64_t)idx[1]) * W", "((int64_t)idx[1]) * W", 1),
    ("no_half_voxel_fp32", "fmaf(u, (float)n, -0.5f)", "fmaf(u, (float)n, 0.0f)", 1),
    ("no_half_voxel_fp64", "(double)u * (double)n - 0.5;", "(double)u * (double)n;", 1),
    ("align_ignored", "(mode & MODE_ALIGN) ? (double)u * (double)(n - 1)", "0 ? (double)u * (double)(n - 1)", 1),
    ("index_x_z_swapped", "((int64_t)idx[2] * H + (int64_t)idx[1]) * W + (int64_t)idx[0]", "((int64_t)idx[0] * H + (int64_t)idx[1]) * W + (int64_t)idx[2]", 1),
    ("upper_border_off_by_one", "idx[a] <= (double)(n[a] - 1)", "idx[a] < (double)(n[a] - 1)", 1),
    ("tent_derivative_sign", "k->dt[a] = up ? 1.0 : -1.0;", "k->dt[a] = up ? -1.0 : 1.0;", 1),
    ("z_grad_scale_uses_h", "A * gd[2] * voxel_scale(s[0], mode)", "A * gd[2] * voxel_scale(s[1], mode)", 1),
    ("x_grad_scale_uses_z", "A * gd[0] * voxel_scale(s[2], mode)", "A * gd[0] * voxel_scale(s[0], mode)", 1),
    ("grad_value_without_A", "double sc = A * t[0] * t[1] * t[2];", "double sc = t[0] * t[1] * t[2];", 1),
    ("grad_z_uses_dx", "gd[2] += t[0] * t[1] * dt[2] * gv;", "gd[2] += dt[0] * t[1] * t[2] * gv;", 1),
    ("forward_drops_z_tent", "double w = A * nb[c].t[0] * nb[c].t[1] * nb[c].t[2];", "double w = A * nb[c].t[0] * nb[c].t[1];", 1),
    ("level_start_ignored", "k->vox = start + ", "k->vox = 0 * start + ", 1),
]


_CHILD = """
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle.volume as ov
from volume_pins import ALL_VOLUME_PINS
orc = ov.VolumeLib({lib!r})
for pin in ALL_VOLUME_PINS:
    try:
        pin(orc)
    except Exception as e:
        print("caught by", pin.__name__, flush=True)
        sys.exit(1)
sys.exit(0)
"""


@pytest.mark.parametrize("name,orig,planted,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_volume_mutant_is_caught(tmp_path, name, orig, planted, count):
    src = open(ov.SRC).read()
    assert src.count(orig) == count, f"mutation site for {name} not found"
    path = tmp_path / "mutant3d.c"
    path.write_text(src.replace(orig, planted))
    lib = ov.build(src=str(path), out=str(tmp_path / f"libmutant3d_{name}.so"))
    # a planted mistake may index outside the arrays: the pins run in a child
    # process, and a pin failure (exit 1) or a crash both count as caught
    tests = os.path.dirname(os.path.abspath(__file__))
    code = _CHILD.format(root=os.path.dirname(tests), tests=tests, lib=lib)
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"no pin caught the planted mistake {name}"
