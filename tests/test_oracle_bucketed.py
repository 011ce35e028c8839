"""Pins of the oracle's bucketed approximate top-k (page "Approximate Top-k
for Increased Parallelism", abstract: many independent small top-k
selections in place of one). Reading: b contiguous buckets of M/b columns,
the exact top-(k/b) of each (lowest column wins ties), listed bucket by
bucket.

The pins check the oracle against: a worked example, the rank definition by
brute force, reductions to textbook routines (b = 1 is the exact top-k;
k = b keeps each bucket's first maximum, numpy's argmax), closed forms, and
the inequality every approximate top-k obeys (its sum never exceeds the exact
top-k's, with equality when the exact top-k is spread evenly).
"""

from __future__ import annotations

import itertools

import numpy as np
import pytest

import oracle


def rank_keep_bucketed(row: np.ndarray, k: int, b: int) -> np.ndarray:
    """Column j survives iff fewer than k/b columns of its own bucket beat
    it (x_i > x_j, or x_i == x_j and i < j)."""
    m = len(row)
    w, keep_n = m // b, k // b
    keep = np.zeros(m, dtype=bool)
    for j in range(m):
        lo = (j // w) * w
        beaten_by = sum(1 for i in range(lo, lo + w)
                        if row[i] > row[j] or (row[i] == row[j] and i < j))
        keep[j] = beaten_by < keep_n
    return keep


def test_worked_example():
    # Buckets [3, 1, 4, 1] and [5, 9, 2, 6]; two survivors each: 3 and 4
    # (columns 0, 2), then 9 and 6 (columns 5, 7).
    x = np.array([[3, 1, 4, 1, 5, 9, 2, 6]], dtype=np.float32)
    v, i = oracle.bucketed(x, 4, 2)
    np.testing.assert_array_equal(i, [[0, 2, 5, 7]])
    np.testing.assert_array_equal(v, [[3, 4, 9, 6]])
    # One survivor per bucket: 4 (column 2) and 9 (column 5). The exact top-2
    # would be 9 and 6: bucketing loses the 6.
    v, i = oracle.bucketed(x, 2, 2)
    np.testing.assert_array_equal(i, [[2, 5]])
    np.testing.assert_array_equal(oracle.exact(x, 2)[1], [[5, 7]])


def test_brute_force_exhaustive_tiny():
    alphabet = [-1.0, 0.0, 2.0]
    for m in range(1, 7):
        rows = np.array(list(itertools.product(alphabet, repeat=m)), dtype=np.float32)
        for b in range(1, m + 1):
            if m % b:
                continue
            for k in range(b, m + 1, b):
                v, i = oracle.bucketed(rows, k, b)
                for r in range(rows.shape[0]):
                    keep = rank_keep_bucketed(rows[r], k, b)
                    np.testing.assert_array_equal(i[r], np.nonzero(keep)[0])
                    np.testing.assert_array_equal(v[r], rows[r][keep])


def test_one_bucket_is_exact():
    rng = np.random.default_rng(21)
    x = (np.round(rng.standard_normal((300, 96)) * 3) / 3).astype(np.float32) + np.float32(0)
    for k in (1, 5, 32, 96):
        ev, ei = oracle.exact(x, k)
        bv, bi = oracle.bucketed(x, k, 1)
        np.testing.assert_array_equal(bi, ei)
        np.testing.assert_array_equal(bv, ev)


def test_one_per_bucket_is_first_argmax():
    rng = np.random.default_rng(22)
    n, m, b = 200, 120, 8
    x = (np.round(rng.standard_normal((n, m)) * 2) / 2).astype(np.float32) + np.float32(0)
    _, i = oracle.bucketed(x, b, b)
    w = m // b
    want = np.argmax(x.reshape(n, b, w), axis=2) + np.arange(b) * w
    np.testing.assert_array_equal(i, want)


def test_k_equals_m_keeps_everything():
    rng = np.random.default_rng(23)
    x = rng.standard_normal((20, 48)).astype(np.float32)
    v, i = oracle.bucketed(x, 48, 6)
    np.testing.assert_array_equal(i, np.tile(np.arange(48), (20, 1)))
    np.testing.assert_array_equal(v, x)


def test_sum_never_exceeds_exact_and_even_spread_is_exact():
    rng = np.random.default_rng(24)
    n, m, k, b = 400, 256, 32, 8
    x = rng.standard_normal((n, m)).astype(np.float32)
    ev, _ = oracle.exact(x, k)
    bv, _ = oracle.bucketed(x, k, b)
    assert np.all(bv.astype(np.float64).sum(1) <= ev.astype(np.float64).sum(1) + 1e-9)
    # Rows whose global top-k has exactly k/b members in every bucket: the
    # bucketed result equals the exact one.
    w = m // b
    y = rng.standard_normal((n, m)).astype(np.float32) - np.float32(10.0)
    for r in range(n):
        for bb in range(b):
            cols = bb * w + rng.choice(w, size=k // b, replace=False)
            y[r, cols] = np.float32(10.0) + rng.random(k // b).astype(np.float32)
    ev, ei = oracle.exact(y, k)
    bv, bi = oracle.bucketed(y, k, b)
    np.testing.assert_array_equal(bi, ei)
    np.testing.assert_array_equal(bv, ev)


@pytest.mark.parametrize("m,k,b", [(10, 4, 3), (12, 5, 2), (8, 4, 0), (8, 9, 1)])
def test_rejects_invalid_buckets(m, k, b):
    with pytest.raises(ValueError):
        oracle.bucketed(np.zeros((2, m), dtype=np.float32), k, b)
