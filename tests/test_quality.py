"""Pins for the approximate-top-k quality figures (row_wise_top_amd/quality.py).

The RTop-K summary page ("Key results", "Experimental setup") reports a hit
rate and max/min relative errors for early stopping without defining them;
quality.py states the definitions used here. These tests hold it to values
worked out by hand from those definitions and to the property every sensible
definition has: an exact top-k scores hit rate 1 and zero errors.
"""

import numpy as np
import pytest

import oracle
import workloads
from row_wise_top_amd.quality import topk_quality


def test_hand_worked_rows():
    # Row 0: exact top-4 = {5, 4, 3, 3} (v_1 = 5, v_k = 3, two copies of 3 in
    # the exact set); selected {5, 3, 2, 1}: above v_k only 5, one copy of 3,
    # so hit = 2/4. relmax = |5 - 5| / 5 = 0, relmin = |1 - 3| / 3 = 2/3.
    # Row 1: exact {8, 6, 4, 2} (v_k = 2, one copy); selected {8, 6, 2, 2}: two
    # copies of v_k but the exact set holds one, so they count once:
    # hit = (2 + 1)/4. relmax = 0, relmin = |2 - 2| / 2 = 0.
    # Row 2: exact {4, 3, 3, 3}; selected {3, 3, 3, 1}: nothing above 3,
    # three copies of v_k = 3 (the exact set has three): hit = 3/4.
    # relmax = |3 - 4| / 4 = 0.25, relmin = |1 - 3| / 3 = 2/3.
    exact = np.array([[5, 4, 3, 3], [8, 6, 4, 2], [4, 3, 3, 3]], dtype=np.float32)
    sel = np.array([[1, 3, 2, 5], [2, 8, 6, 2], [3, 1, 3, 3]], dtype=np.float32)
    q = topk_quality(sel, exact)
    assert q["hit_rate_mean"] == pytest.approx((0.5 + 0.75 + 0.75) / 3)
    assert q["hit_rate_min"] == pytest.approx(0.5)
    assert q["relmax_mean"] == pytest.approx(0.25 / 3)
    assert q["relmax_worst"] == pytest.approx(0.25)
    assert q["relmin_mean"] == pytest.approx((2 / 3 + 0 + 2 / 3) / 3)
    assert q["relmin_worst"] == pytest.approx(2 / 3)
    assert q["relmax_skipped"] == 0 and q["relmin_skipped"] == 0


def test_negative_values_and_tiny_reference():
    # Row 0: exact {-1, -2} (v_1 = -1, v_k = -2); selected {-1, -3}:
    # hit 1/2, relmax 0, relmin |-3 - -2| / 2 = 0.5.
    # Row 1: v_k = 0 exactly: left out of the min-relative error and counted.
    exact = np.array([[-1, -2], [1, 0]], dtype=np.float32)
    sel = np.array([[-3, -1], [0, 1]], dtype=np.float32)
    q = topk_quality(sel, exact)
    assert q["hit_rate_mean"] == pytest.approx((0.5 + 1.0) / 2)
    assert q["relmin_mean"] == pytest.approx(0.5)
    assert q["relmin_skipped"] == 1
    assert q["relmax_skipped"] == 0


@pytest.mark.parametrize("m,k", [(64, 8), (256, 32), (100, 100)])
def test_exact_selection_scores_perfectly(m, k):
    # Any exact top-k (here the oracle's, in any order within a row, ties
    # included) has hit rate 1 and zero relative errors.
    x = np.concatenate([workloads.normal(200, m, 31),
                        workloads.grid_ties(200, m, 32)])
    vals, _ = oracle.exact(x, k)
    rng = np.random.default_rng(0)
    shuffled = np.take_along_axis(vals, rng.permuted(np.tile(np.arange(k), (len(vals), 1)),
                                                     axis=1), axis=1)
    q = topk_quality(shuffled, vals)
    assert q["hit_rate_mean"] == 1.0 and q["hit_rate_min"] == 1.0
    assert q["relmax_worst"] == 0.0 and q["relmin_worst"] == 0.0


def test_capped_quality_improves_with_steps():
    # More search steps can only move the bracket toward v_k: on N(0,1) rows
    # the mean hit rate rises with max_iter and reaches 1 without a cap.
    x = workloads.normal(2000, 256, 33)
    ev, _ = oracle.exact(x, 32)
    hits = [topk_quality(oracle.capped(x, 32, it)[0], ev)["hit_rate_mean"]
            for it in (1, 2, 4, 8)]
    assert hits == sorted(hits)
    assert topk_quality(oracle.capped(x, 32, -1)[0], ev)["hit_rate_mean"] == 1.0


def test_rejects_mismatched_shapes():
    with pytest.raises(ValueError):
        topk_quality(np.zeros((2, 3)), np.zeros((2, 4)))
