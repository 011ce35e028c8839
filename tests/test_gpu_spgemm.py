"""GPU parity of the MaxK-GNN forward aggregation (rtopk_cbsr_spgemm[_u8])
against oracle.spgemm, and of its backward to the compressed features
(rtopk_cbsr_sspmm[_u8]) against oracle.sspmm.

The kernels sum in single precision in an order of their own (forward: LDS
accumulator rows per edge slot, summed at the end, and global float atomics
for rows cut between two waves' edge ranges; backward: global float atomics
per edge), so the bar is the error bound of floating-point summation: every
element must satisfy

    |y_gpu - y_exact| <= (d + 2) * 2^-24 * sum |val * x|  +  2^-126,

with d the row's degree (the number of terms is at most d; each product and
each addition rounds once, relative error u = 2^-24 each, and the bound of a
d-term sum in any order is (d - 1) u over the sum of magnitudes, plus one u
per product and one for the oracle's own rounding of its double sum). The
2^-126 allows for subnormal partial sums flushed by the float atomics.
Everything else (which elements are zero, the shape) must match exactly.

Graphs come from workloads.power_law_graph (seeded); features are the exact
top-k of workload rows as the selection produces them, or random permutations
for k > 64, where a row's survivors take several passes.
"""

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def run_gpu(rp, ci, va, sd, si, m, u8=False):
    import row_wise_top_amd as rt
    d = torch.device("cuda:0")
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).astype(dt)).to(d)
    y = rt.rtopk_cbsr_spgemm(t(rp, np.int64), t(ci, np.int32), t(va, np.float32),
                             t(sd, np.float32), t(si, np.uint8 if u8 else np.int32), m)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def check(rp, ci, va, sd, si, m, label, u8=False):
    want, absum = oracle.spgemm(rp, ci, va, sd.shape[0], sd, si, m, return_absum=True)
    got = run_gpu(rp, ci, va, sd, si, m, u8)
    deg = np.diff(np.asarray(rp, dtype=np.int64)).astype(np.float64)
    tol = (deg[:, None] + 2.0) * 2.0 ** -24 * absum.astype(np.float64) + 2.0 ** -126
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    bad = np.argwhere(err > tol)
    assert bad.size == 0, (f"{label}: {len(bad)} elements outside the bound, first {bad[0]}: "
                           f"got {got[tuple(bad[0])]} want {want[tuple(bad[0])]}")
    # Exact zeros where no term lands.
    assert np.all(got[absum == 0] == 0), f"{label}: nonzero where no term lands"


def features(n_src, m, k, seed, kind="maxk"):
    if kind == "maxk":
        x = workloads.maxk_activation(n_src, m, (seed, seed + 1, seed + 2))
        return oracle.exact(x, k)
    rng = np.random.default_rng(seed)
    sd = rng.standard_normal((n_src, k)).astype(np.float32)
    si = np.stack([rng.permutation(m)[:k] for _ in range(n_src)]).astype(np.int32)
    return sd, si


@pytest.mark.parametrize("n_dst,n_src,mean,cap,m,k", [
    (3000, 2000, 20.0, 500, 256, 32),
    (5000, 5000, 64.0, 4096, 256, 32),
    (2000, 800, 8.0, 100, 128, 16),
    (1500, 1500, 30.0, 1000, 64, 64),
    (1000, 700, 12.0, 300, 1024, 100),
    (800, 600, 10.0, 200, 2048, 300),
    (300, 400, 5.0, 50, 100, 7),
])
def test_power_law_graphs(n_dst, n_src, mean, cap, m, k):
    rp, ci, va = workloads.power_law_graph(n_dst, n_src, mean, cap, seed=n_dst + m)
    sd, si = features(n_src, m, k, seed=7 + k, kind="maxk" if k <= 64 else "perm")
    check(rp, ci, va, sd, si, m, f"int32 {n_dst}x{m} k={k}")
    if m <= 256:
        check(rp, ci, va, sd, si, m, f"u8 {n_dst}x{m} k={k}", u8=True)


def test_one_huge_row_spans_many_waves():
    # Row 3 holds 20,000 edges (about 78 waves' ranges); the rows around it
    # are short and some are empty.
    rng = np.random.default_rng(41)
    deg = np.array([3, 0, 5, 20000, 0, 0, 7, 1, 0, 300])
    rp = np.concatenate([[0], np.cumsum(deg)]).astype(np.int64)
    n_src, m, k = 1000, 256, 32
    ci = rng.integers(0, n_src, size=rp[-1]).astype(np.int32)
    va = rng.standard_normal(rp[-1]).astype(np.float32)
    sd, si = features(n_src, m, k, seed=42)
    check(rp, ci, va, sd, si, m, "huge row")
    check(rp, ci, va, sd, si, m, "huge row u8", u8=True)


def test_many_empty_rows_and_edge_cases():
    n_src, m, k = 50, 64, 8
    sd, si = features(n_src, m, k, seed=43)
    # No edges at all: y is all zero.
    rp = np.zeros(1001, dtype=np.int64)
    check(rp, np.zeros(0, np.int32), np.zeros(0, np.float32), sd, si, m, "no edges")
    # A single edge among many empty rows, at the end.
    rp = np.zeros(701, dtype=np.int64)
    rp[-1] = 1
    check(rp, np.array([3], np.int32), np.array([2.0], np.float32), sd, si, m, "one edge")
    # Rows whose edges start exactly on range boundaries (multiples of 256).
    deg = np.full(40, 256)
    deg[::3] = 0
    rp = np.concatenate([[0], np.cumsum(deg)]).astype(np.int64)
    rng = np.random.default_rng(44)
    ci = rng.integers(0, n_src, size=rp[-1]).astype(np.int32)
    va = rng.random(rp[-1]).astype(np.float32)
    check(rp, ci, va, sd, si, m, "aligned rows")
    # One source row.
    sd1, si1 = sd[:1], si[:1]
    rp, _, va = workloads.power_law_graph(300, 1, 6.0, 40, seed=45)
    check(rp, np.zeros(rp[-1], np.int32), va, sd1, si1, m, "one source row")


def test_out_of_range_edges_and_survivors_are_skipped():
    n_src, m, k = 200, 128, 16
    sd, si = features(n_src, m, k, seed=46, kind="perm")
    si = si.copy()
    si[::7, 3] = m + 5
    si[1::7, 0] = -1
    rp, ci, va = workloads.power_law_graph(900, n_src, 10.0, 120, seed=47)
    ci = ci.copy()
    ci[::11] = n_src + 3
    ci[1::13] = -2
    check(rp, ci, va, sd, si, m, "out of range")


def test_unaligned_features():
    # Features starting one float (one byte) past an aligned address: the
    # kernel's per-lane loads must not assume more alignment than the
    # element size.
    import row_wise_top_amd as rt
    n_src, m, k = 3000, 256, 32
    rp, ci, va = workloads.power_law_graph(2500, n_src, 20.0, 400, seed=49)
    sd, si = features(n_src, m, k, seed=50)
    want, absum = oracle.spgemm(rp, ci, va, n_src, sd, si, m, return_absum=True)
    d = torch.device("cuda:0")
    deg = np.diff(rp).astype(np.float64)
    tol = (deg[:, None] + 2.0) * 2.0 ** -24 * absum.astype(np.float64) + 2.0 ** -126
    for shift in (0, 1):
        bd = torch.zeros(n_src * k + 4, dtype=torch.float32, device=d)
        bd[shift:shift + n_src * k].copy_(torch.from_numpy(sd.reshape(-1)))
        bi = torch.zeros(n_src * k + 4, dtype=torch.uint8, device=d)
        bi[shift:shift + n_src * k].copy_(torch.from_numpy(si.reshape(-1).astype(np.uint8)))
        y = rt.rtopk_cbsr_spgemm(torch.from_numpy(rp).to(d), torch.from_numpy(ci).to(d),
                                 torch.from_numpy(va).to(d),
                                 bd[shift:shift + n_src * k].view(n_src, k),
                                 bi[shift:shift + n_src * k].view(n_src, k), m)
        torch.cuda.synchronize()
        err = np.abs(y.cpu().numpy().astype(np.float64) - want.astype(np.float64))
        assert np.all(err <= tol), f"shift {shift}"


def test_full_size_graph():
    n, m, k = 262144, 256, 32
    rp, ci, va = workloads.power_law_graph(n, n, 64.0, 4096, seed=48)
    x = workloads.config_input(3, n, m)
    sd, si = oracle.exact(x, k)
    check(rp, ci, va, sd, si, m, "262144 nodes, mean degree 64, u8", u8=True)


# --------------------------------------------------------------------------
# Backward to the compressed features (rtopk_cbsr_sspmm[_u8]) against
# oracle.sspmm. Bound: (d + 2) * 2^-24 * sum |terms| + 2^-126 per element,
# d the number of edges into the source row.
# --------------------------------------------------------------------------

def run_gpu_sspmm(rp, ci, va, dy, si, u8=False):
    import row_wise_top_amd as rt
    d = torch.device("cuda:0")
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a).astype(dt)).to(d)
    g = rt.rtopk_cbsr_sspmm(t(rp, np.int64), t(ci, np.int32), t(va, np.float32),
                            t(dy, np.float32), t(si, np.uint8 if u8 else np.int32))
    torch.cuda.synchronize()
    return g.cpu().numpy()


def check_sspmm(rp, ci, va, dy, si, label, u8=False):
    want, absum = oracle.sspmm(rp, ci, va, dy, si, return_absum=True)
    got = run_gpu_sspmm(rp, ci, va, dy, si, u8)
    n_src = si.shape[0]
    ok = (ci >= 0) & (ci < n_src)
    indeg = np.bincount(ci[ok], minlength=n_src).astype(np.float64)
    tol = (indeg[:, None] + 2.0) * 2.0 ** -24 * absum.astype(np.float64) + 2.0 ** -126
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    bad = np.argwhere(err > tol)
    assert bad.size == 0, (f"{label}: {len(bad)} elements outside the bound, first {bad[0]}: "
                           f"got {got[tuple(bad[0])]} want {want[tuple(bad[0])]}")
    assert np.all(got[absum == 0] == 0), f"{label}: nonzero where no term lands"


@pytest.mark.parametrize("n_dst,n_src,mean,cap,m,k", [
    (3000, 2000, 20.0, 500, 256, 32),
    (5000, 5000, 64.0, 4096, 256, 32),
    (2000, 800, 8.0, 100, 128, 16),
    (1000, 700, 12.0, 300, 1024, 100),
    (300, 400, 5.0, 50, 100, 7),
])
def test_sspmm_power_law_graphs(n_dst, n_src, mean, cap, m, k):
    rp, ci, va = workloads.power_law_graph(n_dst, n_src, mean, cap, seed=2 * n_dst + m)
    _, si = features(n_src, m, k, seed=9 + k, kind="maxk" if k <= 64 else "perm")
    dy = workloads.normal(n_dst, m, 70 + m)
    check_sspmm(rp, ci, va, dy, si, f"int32 {n_dst}x{m} k={k}")
    if m <= 256:
        check_sspmm(rp, ci, va, dy, si, f"u8 {n_dst}x{m} k={k}", u8=True)


def test_sspmm_huge_row_and_edge_cases():
    rng = np.random.default_rng(61)
    deg = np.array([3, 0, 5, 20000, 0, 0, 7, 1, 0, 300])
    rp = np.concatenate([[0], np.cumsum(deg)]).astype(np.int64)
    n_src, m, k = 1000, 256, 32
    ci = rng.integers(0, n_src, size=rp[-1]).astype(np.int32)
    va = rng.standard_normal(rp[-1]).astype(np.float32)
    _, si = features(n_src, m, k, seed=62)
    dy = workloads.normal(len(deg), m, 63)
    check_sspmm(rp, ci, va, dy, si, "huge row", u8=True)
    # No edges: every gradient entry is zero.
    rp0 = np.zeros(11, dtype=np.int64)
    check_sspmm(rp0, np.zeros(0, np.int32), np.zeros(0, np.float32), dy, si, "no edges")
    # Out-of-range edges and survivors.
    ci2 = ci.copy()
    ci2[::9] = n_src + 1
    si2 = si.copy()
    si2[::5, 2] = m + 7
    check_sspmm(rp, ci2, va, dy, si2, "out of range")


def test_sspmm_full_size_graph():
    n, m, k = 262144, 256, 32
    rp, ci, va = workloads.power_law_graph(n, n, 64.0, 4096, seed=48)
    _, si = oracle.exact(workloads.config_input(3, n, m), k)
    dy = workloads.normal(n, m, 64)
    check_sspmm(rp, ci, va, dy, si, "262144 nodes, mean degree 64, u8", u8=True)
