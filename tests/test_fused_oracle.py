"""The fused-prologue oracle against its pins, and planted mistakes in copies
of it (CPU only; oracle/fused.py itself is never modified)."""
import importlib.util
import os

import pytest

import oracle
import oracle.fused
from fused_pins import ALL_FUSED_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "fused.py")


@pytest.mark.parametrize("pin", ALL_FUSED_PINS, ids=[p.__name__ for p in ALL_FUSED_PINS])
def test_fused_oracle_pin(pin):
    pin(oracle.fused)


# (name, original text, planted text, count)
MUTANTS = [
    ("normalizer_h_w", "np.stack([s[:, 1], s[:, 0]], axis=-1)", "np.stack([s[:, 0], s[:, 1]], axis=-1)", 1),
    ("offsets_not_divided", "off / nrm[None, None, None, :, None, :]", "off", 1),
    ("offsets_multiplied", "off / nrm[None, None, None, :, None, :]", "off * nrm[None, None, None, :, None, :]", 1),
    ("per_level_ignored", "z.reshape(B, Nq, M, L, K) if per_level else", "z.reshape(B, Nq, M, L, K) if False else", 1),
    ("per_level_always", "z.reshape(B, Nq, M, L, K) if per_level else", "z.reshape(B, Nq, M, L, K) if True else", 1),
    ("level_groups_transposed", "z = z.reshape(B, Nq, M, L, K) if", "z = z.reshape(B, Nq, M, K, L).swapaxes(-1, -2) if", 1),
    ("softmax_no_normalization", "(e / e.sum(axis=-1, keepdims=True))", "e", 1),
    ("grad_offsets_multiplied", "g_off = gl / nrm", "g_off = gl * nrm", 1),
    ("grad_offsets_unscaled", "g_off = gl / nrm[None, None, None, :, None, :]", "g_off = gl", 1),
    ("grad_ref_over_levels", "g_ref = gl.sum(axis=(2, 4))", "g_ref = gl.sum(axis=(2, 4)) * 0 + gl.sum(axis=(2, 3, 4))[:, :, None]", 1),
    ("grad_ref_one_head", "g_ref = gl.sum(axis=(2, 4))", "g_ref = gl[:, :, 0].sum(axis=3)", 1),
    ("grad_logits_no_centering", "(A64 * (gA - s))", "(A64 * gA)", 1),
    ("grad_logits_global_sum_per_level", "s = (A64 * gA).sum(axis=-1, keepdims=True)", "s = (A64 * gA).sum(axis=(-2, -1), keepdims=True)", 1),
    ("grad_logits_no_A", "(A64 * (gA - s))", "(gA - s)", 1),
    # the scale attention S (weights S * A)
    ("scale_ignored", "return A if scale is None else A * np.asarray(scale, dtype=np.float64)", "return A", 1),
    ("scale_squared", "return A if scale is None else A * np.asarray(scale, dtype=np.float64)", "return A if scale is None else A * np.asarray(scale, dtype=np.float64) ** 2", 1),
    ("grad_logits_skip_scale", "gA = S64 * ga", "gA = ga", 1),
    ("grad_scale_without_A", "return gv, g_off, g_logits, g_ref, A64 * ga", "return gv, g_off, g_logits, g_ref, ga", 1),
    ("grad_scale_times_S", "return gv, g_off, g_logits, g_ref, A64 * ga", "return gv, g_off, g_logits, g_ref, S64 * A64 * ga", 1),
    ("grad_scale_of_gA", "return gv, g_off, g_logits, g_ref, A64 * ga", "return gv, g_off, g_logits, g_ref, A64 * gA", 1),
]


def _load_mutant(path, name):
    spec = importlib.util.spec_from_file_location(f"fused_mutant_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,orig,planted,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_fused_mutant_is_caught(tmp_path, name, orig, planted, count):
    src = open(SRC).read()
    assert src.count(orig) == count, f"mutation site for {name} not found"
    path = tmp_path / f"fused_{name}.py"
    path.write_text(src.replace(orig, planted))
    mod = _load_mutant(str(path), name)
    caught = None
    for pin in ALL_FUSED_PINS:
        try:
            pin(mod)
        except Exception:
            caught = pin.__name__
            break
    assert caught is not None, f"no pin caught the planted mistake {name}"
