"""Pins of the oracle's MaxK-GNN forward aggregation Y = A X (review page,
"How MaxK-GNN works"; abstract: row-wise product SpGEMM with the features in
the compressed balanced layout).

The oracle sums with explicit loops in double; the pins check it against a
worked example, numpy's dense float64 matrix product of independently
densified operands, the identity adjacency (Y = dense X exactly), exact
linearity, duplicate edges and empty rows, and the input generator's degree
law.
"""

from __future__ import annotations

import numpy as np

import oracle
import workloads


def dense_x(sp_data, sp_index, m):
    x = np.zeros((sp_data.shape[0], m), dtype=np.float64)
    np.put_along_axis(x, sp_index.astype(np.int64), sp_data.astype(np.float64), axis=1)
    return x


def dense_a(row_ptr, col_idx, val, n_src):
    n = len(row_ptr) - 1
    a = np.zeros((n, n_src), dtype=np.float64)
    rows = np.repeat(np.arange(n), np.diff(row_ptr))
    np.add.at(a, (rows, col_idx.astype(np.int64)), val.astype(np.float64))
    return a


def test_worked_example():
    # Row 0 takes 0.5 * X[0] + 2 * X[1]; row 1 has no edges; row 2 takes -X[1].
    # X[0] = {col 0: 1, col 2: 2}, X[1] = {col 2: 3, col 3: 4}, M = 4.
    rp = np.array([0, 2, 2, 3])
    ci = np.array([0, 1, 1])
    va = np.array([0.5, 2.0, -1.0], dtype=np.float32)
    sd = np.array([[1.0, 2.0], [3.0, 4.0]], dtype=np.float32)
    si = np.array([[0, 2], [2, 3]], dtype=np.int32)
    y = oracle.spgemm(rp, ci, va, 2, sd, si, 4)
    np.testing.assert_array_equal(y, [[0.5, 0, 7, 8], [0, 0, 0, 0], [0, 0, -3, -4]])


def test_matches_dense_product():
    rng = np.random.default_rng(31)
    n_dst, n_src, m, k = 150, 90, 64, 8
    rp, ci, va = workloads.power_law_graph(n_dst, n_src, 12.0, 200, seed=32)
    va = rng.standard_normal(va.shape).astype(np.float32)
    sd = rng.standard_normal((n_src, k)).astype(np.float32)
    si = np.stack([rng.permutation(m)[:k] for _ in range(n_src)]).astype(np.int32)
    y, ab = oracle.spgemm(rp, ci, va, n_src, sd, si, m, return_absum=True)
    a = dense_a(rp, ci, va, n_src)
    x = dense_x(sd, si, m)
    want = a @ x
    # The oracle rounds a double sum once; numpy's product rounds in its own
    # order in double: both agree to float precision.
    np.testing.assert_allclose(y, want, rtol=0, atol=1e-5 * max(1.0, np.abs(want).max()))
    # absum is the sum of |val * x| over edges (duplicates counted per edge).
    a_abs = dense_a(rp, ci, np.abs(va), n_src)
    np.testing.assert_allclose(ab, a_abs @ np.abs(x), rtol=1e-5, atol=1e-6)


def test_identity_adjacency_gives_dense_features():
    rng = np.random.default_rng(33)
    n, m, k = 70, 100, 13
    rp = np.arange(n + 1, dtype=np.int64)
    ci = np.arange(n, dtype=np.int32)
    va = np.ones(n, dtype=np.float32)
    sd = rng.standard_normal((n, k)).astype(np.float32)
    si = np.stack([rng.permutation(m)[:k] for _ in range(n)]).astype(np.int32)
    y = oracle.spgemm(rp, ci, va, n, sd, si, m)
    np.testing.assert_array_equal(y, dense_x(sd, si, m).astype(np.float32))


def test_linearity_duplicates_and_empty_rows():
    rng = np.random.default_rng(34)
    n, m, k = 40, 32, 4
    sd = rng.standard_normal((n, k)).astype(np.float32)
    si = np.stack([rng.permutation(m)[:k] for _ in range(n)]).astype(np.int32)
    # Row 0: neighbour 5 twice; row 1: empty; row 2: neighbour 5 once, weight 2.
    rp = np.array([0, 2, 2, 3], dtype=np.int64)
    ci = np.array([5, 5, 5], dtype=np.int32)
    va = np.array([1.0, 1.0, 2.0], dtype=np.float32)
    y = oracle.spgemm(rp, ci, va, n, sd, si, m)
    np.testing.assert_array_equal(y[0], y[2])
    assert np.all(y[1] == 0)
    rp2, ci2, va2 = workloads.power_law_graph(60, n, 6.0, 30, seed=35)
    y1 = oracle.spgemm(rp2, ci2, va2, n, sd, si, m)
    np.testing.assert_array_equal(oracle.spgemm(rp2, ci2, va2, n, 2 * sd, si, m), 2 * y1)
    np.testing.assert_array_equal(oracle.spgemm(rp2, ci2, 4 * va2, n, sd, si, m), 4 * y1)


def test_out_of_range_entries_are_ignored():
    sd = np.array([[1.0, 2.0], [3.0, 4.0]], dtype=np.float32)
    si = np.array([[0, 9], [1, -1]], dtype=np.int32)  # 9 and -1 lie outside M = 4
    rp = np.array([0, 3], dtype=np.int64)
    ci = np.array([0, 1, 7], dtype=np.int32)          # 7 lies outside n_src = 2
    va = np.ones(3, dtype=np.float32)
    np.testing.assert_array_equal(oracle.spgemm(rp, ci, va, 2, sd, si, 4), [[1, 3, 0, 0]])


def test_generator_degree_law():
    rp, ci, va = workloads.power_law_graph(100000, 50000, 64.0, 4096, seed=36)
    deg = np.diff(rp)
    assert rp[0] == 0 and np.all(deg >= 0) and deg.max() <= 4096
    assert 0.005 < np.mean(deg == 0) < 0.02          # the empty fraction
    assert 50 < deg.mean() < 70                      # near the requested mean
    assert np.all((ci >= 0) & (ci < 50000))
    nz = deg > 0
    np.testing.assert_allclose(np.add.reduceat(va, rp[:-1][nz]), 1.0, rtol=1e-5)
    # Tail: a power law with exponent 2.5 has P(deg >= 4 x_min) = 4**-1.5 = 1/8.
    x_min = 64.0 * 0.5 / 1.5
    tail = np.mean(deg[nz] >= 4 * x_min)
    assert 0.09 < tail < 0.16
