"""Host logic of the parity comparison (tests/parity.py), on hand-made logits.

Each case builds oracle logits and "kernel" logits that differ by less than
the logit bar, then checks that compare_steps accepts exactly the tokens a
correct greedy decoder could emit and rejects the others.
"""
import numpy as np
import pytest

from tests.parity import ABS_TOL, MARGIN, compare_steps


def _case(z_or, noise=None):
    z_or = np.asarray(z_or, np.float32)[None, :]
    z_g = z_or.copy() if noise is None else z_or + np.asarray(noise, np.float32)[None, :]
    return z_g, z_or


def test_clear_winner_must_match():
    z_g, z_o = _case([0.0, 3.0, 1.0, -2.0])
    rep = compare_steps(z_g, np.array([1]), z_o)
    assert rep["pinned"] == 1 and rep["unpinned"] == 0
    # a token that is not the kernel's own first maximum is a broken argmax
    with pytest.raises(AssertionError, match="first maximum"):
        compare_steps(z_g, np.array([2]), z_o)


def test_token_must_be_first_maximum_of_own_logits_on_ties():
    # identical kernel logits at indices 1 and 3: the lowest index wins
    z_g, z_o = _case([0.0, 2.0, 1.0, 2.0])
    compare_steps(z_g, np.array([1]), z_o)
    with pytest.raises(AssertionError, match="first maximum"):
        compare_steps(z_g, np.array([3]), z_o)


def test_near_tie_accepts_either_of_the_top_two():
    # oracle top-2 margin 0.01 < MARGIN: unpinned; the kernel's noise flips them
    z_o = [0.0, 2.0, 1.99, -1.0]
    z_g, z_or = _case(z_o, [0.0, -0.006, 0.006, 0.0])
    rep = compare_steps(z_g, np.array([2]), z_or)
    assert rep["unpinned"] == 1 and rep["pinned"] == 0


def test_unpinned_token_outside_the_bound_is_rejected():
    # the kernel's logits within the bar but its token's oracle logit more than
    # 2 * ABS_TOL below the oracle maximum cannot happen for a correct
    # argmax; planted by giving the kernel a large error at one index
    z_o = np.array([0.0, 2.0, 1.99, 1.9], np.float32)
    z_g = z_o.copy()
    z_g[3] = 2.05                       # error 0.15: fails the logit bar first
    with pytest.raises(AssertionError):
        compare_steps(z_g[None], np.array([3]), z_o[None])


def test_third_logit_far_below_requires_top_two():
    z_o = np.array([0.0, 2.0, 1.99, 1.5], np.float32)
    assert z_o[3] < z_o.max() - 2 * ABS_TOL
    z_g = z_o.copy()
    z_g[3] = 2.1                        # kernel argmax 3, far below in the oracle
    with pytest.raises(AssertionError):
        compare_steps(z_g[None], np.array([3]), z_o[None])


def test_three_way_near_tie_accepts_the_third():
    # top three within 2 * ABS_TOL of each other: a correct kernel may pick any
    z_o = np.array([0.0, 2.0, 1.99, 1.985], np.float32)
    z_g = z_o + np.array([0.0, -0.008, -0.002, 0.009], np.float32)
    assert int(np.argmax(z_g)) == 3
    rep = compare_steps(z_g[None], np.array([3]), z_o[None])
    assert rep["unpinned"] == 1


def test_logit_bar_absolute_and_relative():
    z_o = np.array([0.0, 3.0, 1.0], np.float32)
    compare_steps((z_o + 0.019)[None], np.array([1]), z_o[None])
    with pytest.raises(AssertionError, match="max"):
        compare_steps((z_o + 0.021)[None], np.array([1]), z_o[None])
    # a narrow logit range tightens the bar to 1e-2 of it
    z_n = np.array([0.0, 1.0, 0.5], np.float32)
    with pytest.raises(AssertionError, match="range"):
        compare_steps((z_n + 0.015)[None], np.array([1]), z_n[None])


def test_margin_constant_is_the_stated_bar():
    assert MARGIN == 5e-2 and ABS_TOL == 2e-2
