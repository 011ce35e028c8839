"""Pins for the capped-search oracle (RTop-K summary page, "Approach").

The pages describe the search only in prose and print no worked example, so
the capped replica is pinned by:
  * hand-worked examples (tests/golden/hand_examples.txt), derived from the
    prose by hand;
  * the uncapped search at eps = 0 reaching the exact top-k (ties included),
    a property of any correct bisection with a once-rounded midpoint;
  * closed forms: with no count allowed (max_iter = 0, or eps >= max - min)
    the survivors are the maxima, then the lowest positions of the rest;
  * the midpoint against the exact midpoint rounded once, from rational
    arithmetic, on random brackets including binade crossings, subnormals and
    +-FLT_MAX;
  * the invariants of a valid capped output.
"""

import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from tests.invariants import check_common, check_exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_examples.txt")


def load_golden():
    cases = []
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        row, k, mi, eps, idx, counts = [f.strip() for f in line.split("|")]
        cases.append((np.array([[float(v) for v in row.split()]], dtype=np.float32),
                      int(k), int(mi), float(eps),
                      [int(v) for v in idx.split()], int(counts)))
    return cases


@pytest.mark.parametrize("case", load_golden())
def test_hand_examples(case):
    x, k, max_iter, eps, idx, counts = case
    vals, got_idx, got_counts, lo, hi = oracle.capped(x, k, max_iter, eps, return_state=True)
    assert list(got_idx[0]) == idx
    assert int(got_counts[0]) == counts
    assert (vals[0] == x[0, idx]).all()


def closed_form_no_count(x, k):
    """Survivors when the search performs no count: every position holding the
    row maximum first (lowest positions first, at most k), then the lowest
    remaining positions (all of which lie in [min, max))."""
    n, m = x.shape
    out = np.empty((n, k), dtype=np.int64)
    for r in range(n):
        mx = x[r].max()
        top = [j for j in range(m) if x[r, j] == mx][:k]
        rest = [j for j in range(m) if x[r, j] != mx][: k - len(top)]
        out[r] = sorted(top + rest)
    return out


def all_inputs(m):
    rng = np.random.default_rng(m)
    yield rng.standard_normal((64, m)).astype(np.float32)
    yield rng.integers(-2, 3, size=(64, m)).astype(np.float32)
    yield workloads.adversarial_rows(m)
    yield workloads.grid_ties(32, m, seed=m)
    yield workloads.maxk_activation(32, m, seeds=(m, m + 1, m + 2))


@pytest.mark.parametrize("m", [1, 2, 7, 64, 130, 256])
def test_uncapped_equals_exact(m):
    for x in all_inputs(m):
        for k in sorted({1, max(1, m // 8), max(1, m // 2), m}):
            v_c, i_c = oracle.capped(x, k, -1, 0.0)
            v_e, i_e = oracle.exact(x, k)
            assert (i_c == i_e).all(), (m, k)
            assert (v_c.view(np.uint32) == v_e.view(np.uint32)).all()


@pytest.mark.parametrize("m", [1, 3, 64, 256])
def test_no_count_closed_forms(m):
    for x in all_inputs(m):
        for k in sorted({1, max(1, m // 3), m}):
            _, idx0, c0, _, _ = oracle.capped(x, k, 0, 0.0, return_state=True)
            assert (c0 == 0).all()
            assert (idx0 == closed_form_no_count(x, k)).all()
            span = float(np.max(x.astype(np.float64).max(1) - x.astype(np.float64).min(1)))
            if np.isfinite(span) and span < 3e38:
                eps = np.float32(span) * np.float32(2.0) + np.float32(1.0)
                _, idx1, c1, _, _ = oracle.capped(x, k, -1, float(eps), return_state=True)
                assert (c1 == 0).all()
                assert (idx1 == idx0).all()


def round_to_f32(q: Fraction) -> np.float32:
    """Round a rational to the nearest float32, ties to even (exactly)."""
    if q == 0:
        return np.float32(0.0)
    cand = np.float32(float(q))  # within an ulp or two; fix up exactly below
    best = None
    for c in (np.nextafter(cand, np.float32(-np.inf)), cand,
              np.nextafter(cand, np.float32(np.inf))):
        c = np.float32(c)
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - q)
        even = (int(np.array(c).view(np.uint32)) & 1) == 0
        key = (d, not even)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_midpoint_is_once_rounded():
    rng = np.random.default_rng(7)
    tiny = np.finfo(np.float32).smallest_subnormal
    big = np.finfo(np.float32).max
    pairs = []
    for _ in range(3000):
        e = rng.integers(-150, 128)
        a = np.float32(rng.uniform(-2, 2) * 2.0 ** e) if e < 128 else np.float32(1.0)
        b = np.float32(a + np.float32(rng.uniform(-4, 4)) * np.spacing(np.abs(a)) * rng.integers(1, 1 << 20))
        pairs.append((a, b))
    for _ in range(500):
        pairs.append((np.float32(rng.integers(-50, 50) * tiny), np.float32(rng.integers(-50, 50) * tiny)))
    pairs += [(-big, big), (np.float32(big * 0.75), big), (-big, np.float32(-big * 0.5)),
              (np.float32(-1.0), np.float32(2.0 ** -30)), (np.float32(1.0), np.float32(3.0))]
    checked = 0
    for a, b in pairs:
        if not (np.isfinite(a) and np.isfinite(b)) or a == b:
            continue
        lo, hi = (a, b) if a < b else (b, a)
        x = np.array([[lo, hi]], dtype=np.float32)
        _, _, counts, lo_out, _ = oracle.capped(x, 1, 1, 0.0, return_state=True)
        exact_mid = (Fraction(float(lo)) + Fraction(float(hi))) / 2
        want = round_to_f32(exact_mid)
        halves_exact = (np.float32(lo * np.float32(0.5)) * 2 == lo and
                        np.float32(hi * np.float32(0.5)) * 2 == hi)
        if counts[0] == 1:
            # one count at mid, which selects exactly k = 1: lo = hi = mid.
            assert lo < lo_out[0] < hi
            if halves_exact:
                assert lo_out[0] == want, (lo, hi, lo_out[0], want)
            else:
                assert abs(Fraction(float(lo_out[0])) - exact_mid) <= Fraction(float(tiny))
            checked += 1
        else:
            # no count: the midpoint does not lie strictly inside the bracket
            assert counts[0] == 0
            assert want in (lo, hi) or not halves_exact
    assert checked > 2000


@pytest.mark.parametrize("max_iter", [0, 1, 2, 3, 5, 8])
@pytest.mark.parametrize("eps", [0.0, 1e-4, 0.3])
def test_capped_invariants(max_iter, eps):
    for m in (64, 256, 300):
        for x in all_inputs(m):
            for k in (1, 16, m // 2, m):
                vals, idx, counts, lo, hi = oracle.capped(x, k, max_iter, eps, return_state=True)
                check_common(x, vals, idx, k)
                assert (counts <= max_iter).all()
                # every survivor lies at or above the final lower bound
                assert (vals >= lo[:, None]).all()
                # A = {x >= hi} taken before any fill from [lo, hi)
                n_a = (x >= hi[:, None]).sum(axis=1)
                n_sel_a = (vals >= hi[:, None]).sum(axis=1)
                assert (n_sel_a == np.minimum(n_a, k)).all()
                # the search range always holds at least k elements
                assert ((x >= lo[:, None]).sum(axis=1) >= k).all()


def test_capped_rejects_bad_eps():
    x = np.zeros((1, 4), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.capped(x, 2, -1, -1.0)
    with pytest.raises(ValueError):
        oracle.capped(x, 2, -1, float("nan"))


def test_exactness_of_uncapped_on_config_shapes():
    x = workloads.config_input(1)
    v_e, i_e = oracle.exact(x, 32)
    check_exact(x, v_e, i_e, 32)
    v_c, i_c, counts, _, _ = oracle.capped(x, 32, -1, 0.0, return_state=True)
    assert (i_c == i_e).all()
