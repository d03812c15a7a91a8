"""Plant one mistake at a time in a copy of the oracle (CPU only) and check
that at least one pin catches it.  The copies live in a temporary directory;
oracle/msda_oracle.c itself is never modified."""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "msda_oracle.c")

# (name, original text, planted text, count)
MUTANTS = [
    ("swap_x_y", "neighbours(loc[2 * pt], loc[2 * pt + 1],", "neighbours(loc[2 * pt + 1], loc[2 * pt],", 2),
    ("no_half_pixel_fp32", "fmaf(u, (float)n, -0.5f)", "fmaf(u, (float)n, 0.0f)", 1),
    ("no_half_pixel_fp64", "(double)u * (double)n - 0.5;", "(double)u * (double)n;", 1),
    ("align_corners_true", "fmaf(u, (float)n, -0.5f)", "fmaf(u, (float)(n - 1), 0.0f)", 1),
    ("dwx_sign", "n->dwx = (c & 1) ? 1.0 : -1.0;", "n->dwx = (c & 1) ? -1.0 : 1.0;", 1),
    ("dwy_sign", "n->dwy = (c >> 1) ? 1.0 : -1.0;", "n->dwy = (c >> 1) ? -1.0 : 1.0;", 1),
    ("pixel_index_transposed", "start + (int64_t)yi * W + (int64_t)xi", "start + (int64_t)xi * H + (int64_t)yi", 1),
    ("grad_loc_scale_swapped", "grad_loc[2 * pt] = A * gx * pixel_scale(W, mode);", "grad_loc[2 * pt] = A * gx * pixel_scale(H, mode);", 1),
    ("align_scale_keeps_W", "return (mode & MODE_ALIGN) ? (double)(n - 1) : (double)n;", "return (double)n;", 1),
    ("align_ignored_fp32", "(mode & MODE_ALIGN) ? u * (float)(n - 1) : fmaf", "0 ? u * (float)(n - 1) : fmaf", 1),
    ("align_ignored_fp64", "double p = (mode & MODE_ALIGN) ? (double)u * (double)(n - 1)", "double p = 0 ? (double)u * (double)(n - 1)", 1),
    ("align_with_half_pixel", "? u * (float)(n - 1) : fmaf", "? u * (float)(n - 1) - 0.5f : fmaf", 1),
    ("grad_value_without_A", "double s = A * w;", "double s = w;", 1),
    ("grad_attn_without_tent", "gA += w * gv;", "gA += gv;", 1),
    ("border_off_by_one", "(xi <= (double)(W - 1))", "(xi < (double)(W - 1))", 1),
    ("clamp_instead_of_zero", "if (!inside) {", "if (0) {", 1),
    ("head_offset_dropped", "const float *v = value + ((b * Nv + nb[c].pix) * M + m) * D;", "const float *v = value + ((b * Nv + nb[c].pix) * M) * D;", 1),
    ("level_start_ignored", "n->pix = start + ", "n->pix = 0 * start + ", 1),
    ("grad_y_uses_dwx", "gy += nb[c].wx * nb[c].dwy * gv;", "gy += nb[c].dwx * nb[c].wy * gv;", 1),
]


def _any_pin_fails(orc):
    for pin in ALL_PINS:
        try:
            pin(orc)
        except Exception:
            return pin.__name__
    return None


@pytest.mark.parametrize("name,orig,planted,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, orig, planted, count):
    src = open(SRC).read()
    assert src.count(orig) == count, f"mutation site for {name} not found"
    mutated = src.replace(orig, planted)
    path = tmp_path / "mutant.c"
    path.write_text(mutated)
    lib = oracle.build(src=str(path), out=str(tmp_path / f"libmutant_{name}.so"))
    caught = _any_pin_fails(oracle.OracleLib(lib))
    assert caught is not None, f"no pin caught the planted mistake {name}"
