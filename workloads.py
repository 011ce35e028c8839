"""Seeded synthetic inputs for row-wise top-k.

This module only draws inputs; it holds none of the selection arithmetic. Both
the CPU oracle (through the tests) and the GPU library consume what it returns,
so every comparison runs on identical bytes.

Recipes (numpy ``default_rng`` = PCG64, float32 normals, C-order ``[N, M]``;
every -0.0 is replaced by +0.0 so that the inputs carry a single zero):

* ``normal``          x ~ N(0, 1) i.i.d. (the RTop-K summary page evaluates early
                      stopping on normally distributed synthetic vectors,
                      "Limitations" / "Key results").
* ``maxk_activation`` the MaxK-GNN hidden-activation shape (review page, "How
                      MaxK-GNN works": 256 features per node, k survivors):
                      x = z * s_row with z ~ N(0, 1), a per-row scale
                      s_row ~ U(0.5, 2), and each element set to +0.0 with
                      probability 0.05. Stand-in for the GNN datasets the pages
                      train on, which are not available here.
* ``grid_ties``       x = round(4 z) / 4 with z ~ N(0, 1) (half-to-even
                      rounding): about 30 distinct values per row, so the k-th
                      value is almost always tied.
* ``power_law_graph`` a CSR adjacency for the MaxK-GNN aggregation (review
                      page: feature aggregation over graph edges, evaluated on
                      high-degree graphs that are not available here): row
                      degrees drawn from a power law with exponent 2.5
                      (Pareto, x_min chosen for the requested mean), capped,
                      with a fraction of empty rows; neighbours uniform over
                      the source rows (repeats allowed); edge weight
                      1 / degree of the row (mean aggregation).

Named workloads (rows x row length, k, mode):

====  ===================================================================
 1    1,024 x 256 normal, seed 0, k = 32, exact
 2    65,536 x 256 normal, seed 1, k in {16,32,64,128}, eps in {0,1e-4},
      max_iter in {-1,2,3,4,5}
 3    262,144 x 256 maxk_activation, seeds (2,3,4), k = 32, exact, uint8 idx
 4    16,384 x M in {512,...,8192} grid_ties, seed 5, k in {32,...,256}, exact
 5    1,048,576 x 1,024 normal, seed 6, k = 64, max_iter in {2..8}, eps = 0
====  ===================================================================
"""

from __future__ import annotations

import numpy as np

CONFIG_SEEDS = {1: 0, 2: 1, 3: (2, 3, 4), 4: 5, 5: 6}


def _plus_zero(x: np.ndarray) -> np.ndarray:
    # -0.0 + 0.0 == +0.0 under round-to-nearest; every other value is unchanged.
    x += np.float32(0.0)
    return x


def normal(n: int, m: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return _plus_zero(rng.standard_normal((n, m), dtype=np.float32))


def maxk_activation(n: int, m: int, seeds=(2, 3, 4), zero_prob: float = 0.05
                    ) -> np.ndarray:
    z = np.random.default_rng(seeds[0]).standard_normal((n, m), dtype=np.float32)
    s = np.random.default_rng(seeds[1]).uniform(0.5, 2.0, size=(n, 1)).astype(np.float32)
    zero = np.random.default_rng(seeds[2]).random((n, m), dtype=np.float32) < zero_prob
    z *= s
    z[zero] = np.float32(0.0)
    return _plus_zero(z)


def grid_ties(n: int, m: int, seed: int = 5) -> np.ndarray:
    z = np.random.default_rng(seed).standard_normal((n, m), dtype=np.float32)
    z = np.round(z * np.float32(4.0)) / np.float32(4.0)
    return _plus_zero(z.astype(np.float32))


def config_input(cfg: int, n: int | None = None, m: int | None = None
                 ) -> np.ndarray:
    """The input of a named workload, optionally with fewer rows or another M."""
    if cfg == 1:
        return normal(n or 1024, m or 256, CONFIG_SEEDS[1])
    if cfg == 2:
        return normal(n or 65536, m or 256, CONFIG_SEEDS[2])
    if cfg == 3:
        return maxk_activation(n or 262144, m or 256, CONFIG_SEEDS[3])
    if cfg == 4:
        return grid_ties(n or 16384, m or 1024, CONFIG_SEEDS[4])
    if cfg == 5:
        return normal(n or 1048576, m or 1024, CONFIG_SEEDS[5])
    raise ValueError(f"unknown workload {cfg}")


# --------------------------------------------------------------------------
# Adversarial rows for edge-case parity: each returns a small [N, M] array.
# --------------------------------------------------------------------------

def adversarial_rows(m: int, seed: int = 11) -> np.ndarray:
    """A batch of hand-shaped rows of length m that stress the search.

    Rows: all equal; all equal but one larger / one smaller; a tie block at
    the top; alternating two values; strictly increasing; strictly decreasing;
    tiny subnormal magnitudes around zero; values at +-FLT_MAX; +0/-0 mixes
    (the -0 kept on purpose); a row of adjacent floats; heavy ties at zero;
    and a few normal rows.
    """
    rng = np.random.default_rng(seed)
    f32 = np.float32
    tiny = np.finfo(np.float32).smallest_subnormal
    big = np.finfo(np.float32).max
    rows = []
    rows.append(np.full(m, f32(1.5)))
    r = np.full(m, f32(-2.0)); r[m // 3] = f32(7.0); rows.append(r)
    r = np.full(m, f32(3.0)); r[m // 2] = f32(-1.0); rows.append(r)
    r = rng.standard_normal(m).astype(f32); r[: max(1, m // 4)] = f32(9.0); rows.append(r)
    rows.append(np.where(np.arange(m) % 2 == 0, f32(1.0), f32(2.0)).astype(f32))
    rows.append(np.arange(m, dtype=f32))
    rows.append(np.arange(m, 0, -1).astype(f32))
    rows.append((rng.integers(-4, 5, size=m) * tiny).astype(f32))
    r = rng.choice(np.array([-big, big, f32(0.0), f32(1.0)], dtype=f32), size=m)
    rows.append(r.astype(f32))
    r = rng.choice(np.array([f32(0.0), f32(-0.0), f32(1.0), f32(-1.0)], dtype=f32), size=m)
    rows.append(r.astype(f32))
    base = f32(1.0)
    steps = rng.integers(0, 3, size=m).astype(f32)
    rows.append((base + steps * np.spacing(base)).astype(f32))
    r = np.zeros(m, dtype=f32); r[rng.integers(0, m, size=max(1, m // 8))] = f32(0.5)
    r[rng.integers(0, m, size=max(1, m // 8))] = f32(-0.5); rows.append(r)
    for _ in range(4):
        rows.append(rng.standard_normal(m).astype(f32))
    return np.ascontiguousarray(np.stack(rows).astype(np.float32))


def power_law_graph(n_dst: int, n_src: int, mean_degree: float, max_degree: int,
                    seed: int, exponent: float = 2.5, empty_frac: float = 0.01):
    """(row_ptr int64 [n_dst + 1], col_idx int32 [E], val float32 [E])."""
    rng = np.random.default_rng(seed)
    # Uncapped Pareto mean is x_min * (a - 1) / (a - 2).
    x_min = mean_degree * (exponent - 2.0) / (exponent - 1.0)
    u = rng.random(n_dst)
    deg = np.floor(x_min * (1.0 - u) ** (-1.0 / (exponent - 1.0))).astype(np.int64)
    deg = np.clip(deg, 1, max_degree)
    deg[rng.random(n_dst) < empty_frac] = 0
    row_ptr = np.zeros(n_dst + 1, dtype=np.int64)
    np.cumsum(deg, out=row_ptr[1:])
    nnz = int(row_ptr[-1])
    col_idx = rng.integers(0, n_src, size=nnz, dtype=np.int64).astype(np.int32)
    inv = np.zeros(n_dst, dtype=np.float32)
    inv[deg > 0] = (1.0 / deg[deg > 0]).astype(np.float32)
    val = np.repeat(inv, deg).astype(np.float32)
    return row_ptr, col_idx, val
