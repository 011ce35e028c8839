"""Checks every top-k output must satisfy, independent of how it was produced.

I1 exactly k survivors per row (shape), I2 indices distinct and in [0, M),
I3 each value is bitwise the input at its index, I6 indices ascending,
I4 (exact outputs) every unselected value <= the smallest selected value,
I4b (exact outputs) the selected values are the k largest as a multiset.
"""

from __future__ import annotations

import numpy as np


def check_common(x, vals, idx, k):
    x = np.asarray(x, dtype=np.float32)
    vals = np.asarray(vals, dtype=np.float32)
    idx = np.asarray(idx).astype(np.int64)
    n, m = x.shape
    assert vals.shape == (n, k) and idx.shape == (n, k)            # I1
    assert (idx >= 0).all() and (idx < m).all()                    # I2 range
    if k > 1:
        assert (np.diff(idx, axis=1) > 0).all()                    # I6 + I2 distinct
    gathered = np.take_along_axis(x, idx, axis=1)
    assert (gathered.view(np.uint32) == vals.view(np.uint32)).all()  # I3


def check_exact(x, vals, idx, k):
    check_common(x, vals, idx, k)
    x = np.asarray(x, dtype=np.float32)
    n, m = x.shape
    mask = np.zeros((n, m), dtype=bool)
    np.put_along_axis(mask, np.asarray(idx).astype(np.int64), True, axis=1)
    sel_min = np.asarray(vals).min(axis=1)
    unsel_max = np.where(mask, -np.inf, x).max(axis=1)
    assert (unsel_max <= sel_min).all()                            # I4
    ref = -np.sort(-x, axis=1)[:, :k]
    got = -np.sort(-np.asarray(vals, dtype=np.float32), axis=1)
    assert (ref == got).all()                                      # I4b


def canonical_ties_ok(x, vals, idx, k):
    """Among positions holding the k-th value, the lowest ones were taken."""
    x = np.asarray(x, dtype=np.float32)
    vk = np.asarray(vals).min(axis=1)
    for r in range(x.shape[0]):
        ties = np.flatnonzero(x[r] == vk[r])
        taken = [j for j in idx[r] if x[r, j] == vk[r]]
        if list(taken) != list(ties[: len(taken)]):
            return False
    return True
