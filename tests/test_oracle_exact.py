"""Pins for the exact oracle, independent of its own code.

The exact result is defined by the RTop-K summary page ("Problem": top-k of
each row; unsorted output allowed) and the MaxK-GNN review ("How MaxK-GNN
works": exactly k survivors per node). Ties at the k-th value go to the lowest
indices; survivors are listed in ascending index order.

Pins: exhaustive subset enumeration on every tiny row over a small alphabet
(including -0 and +0), and invariants plus the sorted-value multiset on larger
random and tie-heavy rows.
"""

import itertools

import numpy as np
import pytest

import oracle
import workloads
from tests.invariants import canonical_ties_ok, check_exact


def brute_force_canonical(x: np.ndarray, k: int) -> np.ndarray:
    """Lexicographically first index k-subset whose values all dominate the rest.

    A k-subset is a valid top-k exactly when min(selected) >= max(unselected);
    among valid subsets the lexicographically first sorted index tuple is the
    one that prefers lower indices among tied values.
    """
    n, m = x.shape
    out = np.full((n, k), -1, dtype=np.int64)
    done = np.zeros(n, dtype=bool)
    for combo in itertools.combinations(range(m), k):
        rest = [j for j in range(m) if j not in combo]
        sel_min = x[:, list(combo)].min(axis=1)
        ok = np.ones(n, dtype=bool) if not rest else sel_min >= x[:, rest].max(axis=1)
        new = ok & ~done
        out[new] = combo
        done |= ok
        if done.all():
            break
    assert done.all()
    return out


@pytest.mark.parametrize("m", [1, 2, 3, 4, 5, 6])
def test_exhaustive_small_rows(m):
    alphabet = np.array([-1.0, -0.0, 0.0, 1.0, 2.0], dtype=np.float32)
    rows = np.array(list(itertools.product(range(len(alphabet)), repeat=m)))
    x = alphabet[rows].astype(np.float32)
    for k in range(1, m + 1):
        vals, idx = oracle.exact(x, k)
        expect = brute_force_canonical(x, k)
        assert (idx == expect).all(), f"m={m} k={k}"
        gathered = np.take_along_axis(x, expect, axis=1)
        assert (vals.view(np.uint32) == gathered.view(np.uint32)).all()


@pytest.mark.parametrize("m,k", [(7, 3), (8, 8), (16, 5), (33, 1), (64, 17), (64, 64), (200, 32)])
def test_random_rows_invariants(m, k):
    rng = np.random.default_rng(m * 100 + k)
    x_norm = rng.standard_normal((300, m)).astype(np.float32)
    x_ties = rng.integers(-3, 4, size=(300, m)).astype(np.float32)
    for x in (x_norm, x_ties):
        vals, idx = oracle.exact(x, k)
        check_exact(x, vals, idx, k)
        assert canonical_ties_ok(x, vals, idx, k)


def test_adversarial_rows():
    for m in (1, 5, 64, 100, 256):
        x = workloads.adversarial_rows(m)
        for k in sorted({1, max(1, m // 2), m}):
            vals, idx = oracle.exact(x, k)
            check_exact(x, vals, idx, k)
            assert canonical_ties_ok(x, vals, idx, k)


def test_rejects_bad_arguments():
    x = np.zeros((2, 4), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.exact(x, 0)
    with pytest.raises(ValueError):
        oracle.exact(x, 5)


def test_thread_count_does_not_change_results():
    # The baseline timing runs the oracle on all host threads and on one.
    x = workloads.normal(3000, 256, 17)
    before = oracle.threads()
    want = oracle.exact(x, 32)
    oracle.set_threads(1)
    try:
        assert oracle.threads() == 1
        got = oracle.exact(x, 32)
    finally:
        oracle.set_threads(before)
    assert oracle.threads() == before
    assert np.array_equal(got[1], want[1])
    assert np.array_equal(got[0].view(np.uint32), want[0].view(np.uint32))
    with pytest.raises(ValueError):
        oracle.set_threads(0)
