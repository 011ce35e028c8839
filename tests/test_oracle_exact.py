"""Pins for the exact oracle, independent of its own code.

The exact result is defined by the RTop-K summary page ("Problem": top-k of
each row; unsorted output allowed) and the MaxK-GNN review ("How MaxK-GNN
works": exactly k survivors per node). Ties at the k-th value go to the lowest
indices; survivors are listed in ascending index order.

Pins: exhaustive subset enumeration on every tiny row over a small alphabet
(including -0 and +0), and invariants plus the sorted-value multiset on larger
random and tie-heavy rows. The oracle's partial-selection path
(``oracle.exact``, std::nth_element) and its full stable-sort path
(``oracle.exact_by_sort``) are both held to these pins and to each other.
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
        expect = brute_force_canonical(x, k)
        gathered = np.take_along_axis(x, expect, axis=1)
        for path in (oracle.exact, oracle.exact_by_sort):
            vals, idx = path(x, k)
            assert (idx == expect).all(), f"{path.__name__} m={m} k={k}"
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


@pytest.mark.parametrize("m", [1, 7, 64, 256, 1000, 4096])
def test_partial_selection_equals_stable_sort(m):
    # Two independent computations of the same definition must agree bit for
    # bit (indices and value bits), ties and signed zeros included.
    rng = np.random.default_rng(m)
    families = [
        rng.standard_normal((200, m)).astype(np.float32),
        rng.integers(-2, 3, size=(200, m)).astype(np.float32),
        np.round(4 * rng.standard_normal((200, m))).astype(np.float32) / 4,
        np.where(rng.random((200, m)) < 0.5, np.float32(-0.0), np.float32(0.0)),
        workloads.adversarial_rows(m),
    ]
    for x in families:
        for k in sorted({1, max(1, m // 3), max(1, m - 1), m}):
            a = oracle.exact(x, k)
            b = oracle.exact_by_sort(x, k)
            assert np.array_equal(a[1], b[1]), f"m={m} k={k}"
            assert np.array_equal(a[0].view(np.uint32), b[0].view(np.uint32))


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
