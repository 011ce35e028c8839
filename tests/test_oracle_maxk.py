"""Pins of the oracle's MaxK nonlinearity (MaxK-GNN review, "How MaxK-GNN
works": each row keeps exactly its k largest features, the rest become zero,
and only the survivors carry gradient back through the same sp_index).

Each pin checks the oracle against something other than itself: a worked
example, the rank definition evaluated by brute force, closed forms and
symmetries, the adjoint identity of gather and scatter, and a finite
difference of the forward function.
"""

from __future__ import annotations

import itertools

import numpy as np
import pytest

import oracle


def rank_keep(row: np.ndarray, k: int) -> np.ndarray:
    """Column j survives iff fewer than k columns beat it, where column i
    beats j when x_i > x_j, or x_i == x_j and i < j (lowest index wins)."""
    m = len(row)
    keep = np.zeros(m, dtype=bool)
    for j in range(m):
        beaten_by = 0
        for i in range(m):
            if row[i] > row[j] or (row[i] == row[j] and i < j):
                beaten_by += 1
        keep[j] = beaten_by < k
    return keep


def test_worked_example():
    # x = [3, 1, 4, 1, 5, 9, 2, 6], k = 3: the three largest are 9, 6, 5 at
    # columns 5, 7, 4; everything else becomes zero.
    x = np.array([[3, 1, 4, 1, 5, 9, 2, 6]], dtype=np.float32)
    y, vals, idx = oracle.maxk_forward(x, 3)
    np.testing.assert_array_equal(y, [[0, 0, 0, 0, 5, 9, 0, 6]])
    np.testing.assert_array_equal(vals, [[5, 9, 6]])
    np.testing.assert_array_equal(idx, [[4, 5, 7]])
    # The gradient of the three survivors goes back to columns 4, 5, 7.
    g = np.array([[10, 20, 30]], dtype=np.float32)
    np.testing.assert_array_equal(oracle.maxk_backward(g, idx, 8),
                                  [[0, 0, 0, 0, 10, 20, 0, 30]])


def test_brute_force_exhaustive_tiny():
    alphabet = [-1.0, 0.0, 1.0, 2.0]
    for m in range(1, 6):
        rows = np.array(list(itertools.product(alphabet, repeat=m)), dtype=np.float32)
        for k in range(1, m + 1):
            y, vals, idx = oracle.maxk_forward(rows, k)
            for r in range(rows.shape[0]):
                keep = rank_keep(rows[r], k)
                np.testing.assert_array_equal(y[r], np.where(keep, rows[r], 0.0))
                np.testing.assert_array_equal(idx[r], np.nonzero(keep)[0])
                np.testing.assert_array_equal(vals[r], rows[r][keep])


def test_k_equals_m_is_identity_and_k1_keeps_first_max():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((50, 37), dtype=np.float32)
    y, _, _ = oracle.maxk_forward(x, 37)
    np.testing.assert_array_equal(y, x)
    x[:, 5] = 4.0
    x[:, 20] = 4.0  # two equal maxima: the lower column wins at k = 1
    y, vals, idx = oracle.maxk_forward(x, 1)
    assert np.all(idx[:, 0] == 5)
    expect = np.zeros_like(x)
    expect[:, 5] = 4.0
    np.testing.assert_array_equal(y, expect)


def test_scale_and_permutation_equivariance():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((40, 64), dtype=np.float32)  # distinct values
    k = 9
    y, _, _ = oracle.maxk_forward(x, k)
    y2, _, _ = oracle.maxk_forward(2.0 * x, k)  # exact scaling by 2
    np.testing.assert_array_equal(y2, 2.0 * y)
    perm = rng.permutation(64)
    yp, _, _ = oracle.maxk_forward(x[:, perm], k)
    np.testing.assert_array_equal(yp, y[:, perm])


def test_backward_is_adjoint_of_gather():
    # <scatter(g, idx), d> == <g, gather(d, idx)> for every d: the backward
    # is the transpose of taking the survivors. N, M, k all differ so that a
    # transposed index fails.
    rng = np.random.default_rng(13)
    n, m, k = 23, 41, 7
    idx = np.stack([rng.permutation(m)[:k] for _ in range(n)]).astype(np.int32)
    g = rng.standard_normal((n, k)).astype(np.float32)
    d = rng.standard_normal((n, m))
    gx = oracle.maxk_backward(g, idx, m).astype(np.float64)
    lhs = float((gx * d).sum())
    rhs = float((g.astype(np.float64) * np.take_along_axis(d, idx, axis=1)).sum())
    assert abs(lhs - rhs) <= 1e-9 * max(1.0, abs(rhs))
    # Columns that no index names stay exactly zero.
    named = np.zeros((n, m), dtype=bool)
    np.put_along_axis(named, idx, True, axis=1)
    assert np.all(gx[~named] == 0.0)


def test_backward_matches_finite_difference_of_forward():
    # L(x) = sum(w * maxk(x)). Rows with well separated values keep their
    # selection under a small perturbation, so the central difference of L
    # along d equals <grad_x, d> with grad_x = backward(gather(w, idx)).
    rng = np.random.default_rng(14)
    n, m, k = 16, 48, 6
    base = np.stack([rng.permutation(m) for _ in range(n)]).astype(np.float64)
    x = (base * 0.5).astype(np.float32)  # gaps of 0.5 between values
    w = rng.standard_normal((n, m)).astype(np.float32)
    d = rng.standard_normal((n, m)).astype(np.float32)
    eps = np.float32(2.0 ** -8)

    def loss(z):
        y, _, _ = oracle.maxk_forward(z, k)
        return float((w.astype(np.float64) * y.astype(np.float64)).sum())

    fd = (loss(x + eps * d) - loss(x - eps * d)) / (2.0 * float(eps))
    _, _, idx = oracle.maxk_forward(x, k)
    gx = oracle.maxk_backward(np.take_along_axis(w, idx, axis=1), idx, m)
    analytic = float((gx.astype(np.float64) * d.astype(np.float64)).sum())
    assert abs(fd - analytic) <= 1e-4 * max(1.0, abs(analytic))


def test_backward_ignores_out_of_range_indices():
    g = np.array([[1.0, 2.0, 3.0]], dtype=np.float32)
    idx = np.array([[-1, 2, 5]], dtype=np.int32)  # only column 2 is in [0, 5)
    np.testing.assert_array_equal(oracle.maxk_backward(g, idx, 5), [[0, 0, 2.0, 0, 0]])


def test_forward_survivors_agree_with_exact():
    rng = np.random.default_rng(15)
    x = np.round(rng.standard_normal((200, 100)) * 2) / 2  # many ties
    x = x.astype(np.float32) + np.float32(0.0)
    for k in (1, 7, 50, 100):
        _, vals, idx = oracle.maxk_forward(x, k)
        ev, ei = oracle.exact(x, k)
        np.testing.assert_array_equal(vals, ev)
        np.testing.assert_array_equal(idx, ei)


@pytest.mark.parametrize("m,k", [(0, 3), (4, 5), (3, 0)])
def test_forward_rejects_invalid_k(m, k):
    with pytest.raises(ValueError):
        oracle.maxk_forward(np.zeros((2, m), dtype=np.float32), k)
