"""Pins of the oracle's backward of the MaxK-GNN aggregation with respect to
the compressed features (review page: the backward samples exactly the
sp_index positions, reusing the forward's pattern): grad_sp[j, t] =
(A^T dY)[j, sp_index[j, t]].

Pins: a worked example; numpy's dense float64 product A^T dY sampled at the
survivors; the adjoint identity <A X(s), dY> = <s, grad_sp> for the forward
oracle (pinned on its own), which fixes the backward as the transpose of the
forward map s -> A X(s); a central finite difference of the forward; and
exact linearity.
"""

from __future__ import annotations

import numpy as np

import oracle
import workloads


def dense_a(row_ptr, col_idx, val, n_src):
    n = len(row_ptr) - 1
    a = np.zeros((n, n_src), dtype=np.float64)
    rows = np.repeat(np.arange(n), np.diff(row_ptr))
    np.add.at(a, (rows, col_idx.astype(np.int64)), val.astype(np.float64))
    return a


def test_worked_example():
    # Edges: row 0 -> src 0 (0.5), row 0 -> src 1 (2), row 2 -> src 1 (-1).
    # src 0 keeps columns {0, 2}; src 1 keeps {2, 3}. dY rows r0, r1, r2.
    rp = np.array([0, 2, 2, 3])
    ci = np.array([0, 1, 1])
    va = np.array([0.5, 2.0, -1.0], dtype=np.float32)
    si = np.array([[0, 2], [2, 3]], dtype=np.int32)
    dy = np.array([[1, 2, 3, 4], [5, 6, 7, 8], [9, 10, 11, 12]], dtype=np.float32)
    g = oracle.sspmm(rp, ci, va, dy, si)
    # src 0: 0.5 * r0 at (0, 2) = (0.5, 1.5)
    # src 1: 2 * r0 at (2, 3) - r2 at (2, 3) = (6 - 11, 8 - 12) = (-5, -4)
    np.testing.assert_array_equal(g, [[0.5, 1.5], [-5.0, -4.0]])


def test_matches_dense_transpose_product():
    rng = np.random.default_rng(51)
    n_dst, n_src, m, k = 140, 90, 48, 6
    rp, ci, va = workloads.power_law_graph(n_dst, n_src, 10.0, 150, seed=52)
    va = rng.standard_normal(va.shape).astype(np.float32)
    dy = rng.standard_normal((n_dst, m)).astype(np.float32)
    si = np.stack([rng.permutation(m)[:k] for _ in range(n_src)]).astype(np.int32)
    g = oracle.sspmm(rp, ci, va, dy, si)
    full = dense_a(rp, ci, va, n_src).T @ dy.astype(np.float64)
    want = np.take_along_axis(full, si.astype(np.int64), axis=1)
    np.testing.assert_allclose(g, want, rtol=0, atol=1e-5 * max(1.0, np.abs(want).max()))


def test_adjoint_of_the_forward():
    rng = np.random.default_rng(53)
    n_dst, n_src, m, k = 200, 150, 64, 8
    rp, ci, va = workloads.power_law_graph(n_dst, n_src, 12.0, 200, seed=54)
    s = rng.standard_normal((n_src, k)).astype(np.float32)
    si = np.stack([rng.permutation(m)[:k] for _ in range(n_src)]).astype(np.int32)
    dy = rng.standard_normal((n_dst, m)).astype(np.float32)
    y = oracle.spgemm(rp, ci, va, n_src, s, si, m)
    g = oracle.sspmm(rp, ci, va, dy, si)
    lhs = float((y.astype(np.float64) * dy).sum())
    rhs = float((s.astype(np.float64) * g).sum())
    assert abs(lhs - rhs) <= 1e-5 * max(1.0, abs(lhs))


def test_finite_difference_of_the_forward():
    rng = np.random.default_rng(55)
    n_dst, n_src, m, k = 60, 40, 32, 4
    rp, ci, va = workloads.power_law_graph(n_dst, n_src, 6.0, 40, seed=56)
    s = rng.standard_normal((n_src, k)).astype(np.float32)
    si = np.stack([rng.permutation(m)[:k] for _ in range(n_src)]).astype(np.int32)
    w = rng.standard_normal((n_dst, m)).astype(np.float32)
    d = rng.standard_normal((n_src, k)).astype(np.float32)
    eps = np.float32(2.0 ** -6)

    def loss(z):
        return float((oracle.spgemm(rp, ci, va, n_src, z, si, m).astype(np.float64) * w).sum())

    fd = (loss(s + eps * d) - loss(s - eps * d)) / (2.0 * float(eps))
    g = oracle.sspmm(rp, ci, va, w, si)
    assert abs(fd - float((g.astype(np.float64) * d).sum())) <= 1e-3 * max(1.0, abs(fd))


def test_linearity_and_ignored_entries():
    rng = np.random.default_rng(57)
    n_dst, n_src, m, k = 50, 30, 16, 4
    rp, ci, va = workloads.power_law_graph(n_dst, n_src, 5.0, 30, seed=58)
    si = np.stack([rng.permutation(m)[:k] for _ in range(n_src)]).astype(np.int32)
    dy = rng.standard_normal((n_dst, m)).astype(np.float32)
    g = oracle.sspmm(rp, ci, va, dy, si)
    np.testing.assert_array_equal(oracle.sspmm(rp, ci, 2 * va, dy, si), 2 * g)
    np.testing.assert_array_equal(oracle.sspmm(rp, ci, va, 4 * dy, si), 4 * g)
    ci2 = ci.copy()
    ci2[::5] = n_src + 2   # edges to a missing source row contribute nothing
    si2 = si.copy()
    si2[:, 0] = m + 1      # a survivor outside M gets nothing
    g2 = oracle.sspmm(rp, ci2, va, dy, si2)
    assert np.all(g2[:, 0] == 0)
