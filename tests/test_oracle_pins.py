"""The CPU oracle against its pins (no GPU): see tests/oracle_pins.py."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


@pytest.mark.parametrize("align", [0, oracle.ALIGN], ids=["half_pixel", "align_corners"])
def test_spec_and_double_modes_agree(orc, align):
    """The fp32 coordinate transform and the fp64 one give the same forward
    to ~1e-6 on the tiny config (their difference is coordinate rounding), in
    either pixel convention."""
    import workloads
    from oracle_pins import max_rel
    w = workloads.make(0)
    a = orc.forward(w.value, w.spatial_shapes, w.level_start_index, w.sampling_loc,
                    w.attn_weight, mode=oracle.SPEC | align)
    b = orc.forward(w.value, w.spatial_shapes, w.level_start_index, w.sampling_loc,
                    w.attn_weight, mode=oracle.DOUBLE | align)
    assert max_rel(a, b) < 1e-6


def test_thread_count_does_not_change_results(orc):
    import numpy as np
    import workloads
    w = workloads.random_case(5, 3, ((9, 7), (5, 4)), 40, 4, 8, 4)
    args = (w.value, w.spatial_shapes, w.level_start_index, w.sampling_loc, w.attn_weight)
    assert np.array_equal(orc.forward(*args, threads=1), orc.forward(*args, threads=4))
    b1 = orc.backward(*args, w.grad_out, threads=1)
    b4 = orc.backward(*args, w.grad_out, threads=4)
    for x, y in zip(b1, b4):
        assert np.array_equal(x, y)


def test_rejects_inconsistent_level_table(orc):
    import numpy as np
    import workloads
    w = workloads.random_case(6, 1, ((4, 4), (2, 2)), 3, 1, 4, 2)
    bad_start = np.array([0, 15], dtype=np.int64)
    with pytest.raises(ValueError):
        orc.forward(w.value, w.spatial_shapes, bad_start, w.sampling_loc, w.attn_weight)
