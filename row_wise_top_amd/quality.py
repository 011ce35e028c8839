"""Quality of an approximate (early-stopped) top-k against the exact one.

The RTop-K summary page ("Key results", "Experimental setup") reports hit rate
and max/min relative error for early stopping without defining them. The
definitions used here:

* hit rate of a row: the size of the multiset intersection of the selected
  values with the exact top-k values, over k. Every selected value above the
  exact k-th value v_k counts; values equal to v_k count up to the number of
  copies of v_k in the exact set.
* max relative error: |max(selected) - v_1| / |v_1|, v_1 the row maximum.
* min relative error: |min(selected) - v_k| / |v_k|.

Rows whose reference value has magnitude below ``tiny`` are left out of the
relative errors and counted in ``*_skipped``.
"""

from __future__ import annotations

import numpy as np


def topk_quality(selected_vals, exact_vals, tiny: float = 1e-6) -> dict:
    sel = np.asarray(selected_vals, dtype=np.float64)
    ex = np.asarray(exact_vals, dtype=np.float64)
    if sel.shape != ex.shape or sel.ndim != 2:
        raise ValueError("selected and exact values must both be [N, k]")
    k = sel.shape[1]
    v1 = ex.max(axis=1)
    vk = ex.min(axis=1)
    n_gt = (sel > vk[:, None]).sum(axis=1)
    n_eq = np.minimum((sel == vk[:, None]).sum(axis=1),
                      (ex == vk[:, None]).sum(axis=1))
    hit = (n_gt + n_eq) / k
    ok1 = np.abs(v1) >= tiny
    okk = np.abs(vk) >= tiny
    relmax = np.abs(sel.max(axis=1) - v1)[ok1] / np.abs(v1[ok1])
    relmin = np.abs(sel.min(axis=1) - vk)[okk] / np.abs(vk[okk])
    return {
        "hit_rate_mean": float(hit.mean()) if hit.size else 1.0,
        "hit_rate_min": float(hit.min()) if hit.size else 1.0,
        "relmax_mean": float(relmax.mean()) if relmax.size else 0.0,
        "relmax_worst": float(relmax.max()) if relmax.size else 0.0,
        "relmin_mean": float(relmin.mean()) if relmin.size else 0.0,
        "relmin_worst": float(relmin.max()) if relmin.size else 0.0,
        "relmax_skipped": int((~ok1).sum()),
        "relmin_skipped": int((~okk).sum()),
    }
