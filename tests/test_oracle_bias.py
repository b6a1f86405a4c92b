"""Pins of the oracle's load-balancing bias update (auxiliary-loss-free balancing of
DeepSeek-V3, arXiv:2412.19437 §2.1.2): closed-form cases, exact ties at the mean, and the
fp32 rounding of the update."""
import numpy as np
import pytest

import oracle as orc


def test_over_and_under_loaded_move_opposite_ways():
    b = orc.update_bias([3, 1], [0.0, 0.0], 0.25)
    assert b.tolist() == [-0.25, 0.25]


def test_equal_loads_leave_bias_unchanged():
    b0 = np.array([0.5, -1.0, 2.0, 0.0], np.float32)
    assert np.array_equal(orc.update_bias([5, 5, 5, 5], b0, 0.1), b0)


def test_expert_exactly_at_the_mean_is_unchanged():
    # total 6 over 3 experts: mean 2, so expert 1 sits exactly on it
    b = orc.update_bias([1, 2, 3], [0.0, 0.0, 0.0], 1.0)
    assert b.tolist() == [1.0, 0.0, -1.0]


def test_mean_is_not_rounded():
    # total 7 over 3 experts: mean 7/3; a count of 2 is below it, 3 above (2*3 < 7 < 3*3)
    b = orc.update_bias([2, 3, 2], [0.0, 0.0, 0.0], 0.5)
    assert b.tolist() == [0.5, -0.5, 0.5]


def test_empty_and_all_on_one_expert():
    b = orc.update_bias([0, 0, 8, 0], [0.0] * 4, 0.125)
    assert b.tolist() == [0.125, 0.125, -0.125, 0.125]
    assert orc.update_bias([0, 0], [1.0, 2.0], 0.3).tolist() == [1.0, 2.0]


def test_update_is_one_fp32_rounding():
    # 1 + 2^-25 is not representable in fp32 and rounds back to 1 (ties to even)
    b = orc.update_bias([0, 4], [1.0, 1.0], 2.0 ** -25)
    assert b.dtype == np.float32 and b[0] == np.float32(1.0) and b[1] == np.float32(1.0)
    # 1 + 3*2^-25 rounds up to 1 + 2^-23; 1 - 3*2^-25 lies halfway between 1 - 2^-24 and
    # 1 - 2^-23 (spacing 2^-24 below 1) and ties to the even one, 1 - 2^-23
    b = orc.update_bias([0, 4], [1.0, 1.0], 3 * 2.0 ** -25)
    assert b[0] == np.float32(1.0 + 2.0 ** -23)
    assert b[1] == np.float32(1.0 - 2.0 ** -23)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_brute_force_sign_rule(seed):
    rs = np.random.default_rng(seed)
    E = 64
    counts = rs.integers(0, 50, size=E).astype(np.int32)
    bias = rs.normal(size=E).astype(np.float32)
    g = np.float32(0.001)
    got = orc.update_bias(counts, bias, float(g))
    mean = counts.sum() / E  # float compare is exact here: counts and E are small
    for e in range(E):
        want = bias[e] if counts[e] == mean else (bias[e] - g if counts[e] > mean else bias[e] + g)
        assert got[e] == np.float32(want)
