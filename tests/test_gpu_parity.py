"""GPU parity: the HIP kernels against the CPU oracle, bit for bit.

Selection does no arithmetic on the values it returns, so the bar is exact
identity: the same column indices and the same value bits as the oracle, for
the exact mode (lowest index wins ties on both sides) and for the capped
search with the same max_iter / eps. Inputs come from workloads.py (seeded);
every expected value comes from oracle/.

Workloads: the five named shapes at full size (every row of the 4 GiB one
too), adversarial rows at many row
lengths (ties, +-0, subnormals, +-FLT_MAX, constant rows), ragged row counts,
and guard bands around the outputs.
"""

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def rt():
    import row_wise_top_amd
    return row_wise_top_amd


def dev():
    return torch.device("cuda:0")


def gpu_run(x_np, k, mode, max_iter=-1, eps=0.0, u8=False):
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to(dev())
    return gpu_run_t(x, k, mode, max_iter, eps, u8)


def gpu_run_t(x, k, mode, max_iter=-1, eps=0.0, u8=False):
    r = rt()
    if mode == "exact":
        v, i = (r.rtopk_select_exact_u8 if u8 else r.rtopk_select_exact)(x, k)
    else:
        v, i = (r.rtopk_select_u8 if u8 else r.rtopk_select)(x, k, max_iter, eps)
    torch.cuda.synchronize()
    return v.cpu().numpy(), i.cpu().numpy().astype(np.int32)


def oracle_run(x_np, k, mode, max_iter=-1, eps=0.0):
    if mode == "exact":
        return oracle.exact(x_np, k)
    return oracle.capped(x_np, k, max_iter, eps)


def assert_identical(got, want, label):
    gv, gi = got
    wv, wi = want
    bad_rows = np.flatnonzero((gi != wi).any(axis=1) |
                              (gv.view(np.uint32) != wv.view(np.uint32)).any(axis=1))
    assert bad_rows.size == 0, (
        f"{label}: {bad_rows.size} rows differ, first {bad_rows[:5].tolist()}; "
        f"row {bad_rows[0]}: got idx {gi[bad_rows[0]][:16].tolist()} "
        f"want {wi[bad_rows[0]][:16].tolist()}")


def check(x_np, k, mode, max_iter=-1, eps=0.0, u8=False, label=""):
    print(f"[parity] {label} N={x_np.shape[0]} M={x_np.shape[1]} k={k} {mode} "
          f"max_iter={max_iter} eps={eps} u8={u8}", flush=True)
    got = gpu_run(x_np, k, mode, max_iter, eps, u8)
    want = oracle_run(x_np, k, mode, max_iter, eps)
    assert_identical(got, want, label)


# ---------------------------------------------------------------------------
# Named workloads
# ---------------------------------------------------------------------------

def test_workload1_exact_and_uncapped():
    x = workloads.config_input(1)
    for u8 in (False, True):
        check(x, 32, "exact", u8=u8, label="w1")
        check(x, 32, "capped", -1, 0.0, u8=u8, label="w1-uncapped")


@pytest.fixture(scope="module")
def w2():
    return workloads.config_input(2)


@pytest.mark.parametrize("k", [16, 32, 64, 128])
def test_workload2_sweep(w2, k):
    x = torch.from_numpy(w2).to(dev())
    print(f"[parity] w2 k={k} exact", flush=True)
    assert_identical(gpu_run_t(x, k, "exact"), oracle.exact(w2, k), f"w2 exact k={k}")
    for eps in (0.0, 1e-4):
        for max_iter in (-1, 2, 3, 4, 5):
            print(f"[parity] w2 k={k} eps={eps} max_iter={max_iter}", flush=True)
            got = gpu_run_t(x, k, "capped", max_iter, eps)
            want = oracle.capped(w2, k, max_iter, eps)
            assert_identical(got, want, f"w2 k={k} eps={eps} max_iter={max_iter}")


def test_workload3_full_size():
    x = workloads.config_input(3)
    print("[parity] w3 full 262144x256 exact u8", flush=True)
    xt = torch.from_numpy(x).to(dev())
    want = oracle.exact(x, 32)
    assert_identical(gpu_run_t(xt, 32, "exact", u8=True), want, "w3 exact u8")
    assert_identical(gpu_run_t(xt, 32, "exact", u8=False), want, "w3 exact i32")
    assert_identical(gpu_run_t(xt, 32, "capped", -1, 0.0, u8=True), want, "w3 uncapped u8")
    # The early-stopped search at full size (the benchmarked settings).
    for mi in (2, 4):
        print(f"[parity] w3 full capped max_iter={mi} u8", flush=True)
        assert_identical(gpu_run_t(xt, 32, "capped", mi, 0.0, u8=True),
                         oracle.capped(x, 32, mi, 0.0), f"w3 capped {mi} u8")


@pytest.mark.parametrize("m", [512, 1024, 2048, 4096, 8192])
def test_workload4_ties(m):
    x = workloads.config_input(4, m=m)
    xt = torch.from_numpy(x).to(dev())
    for k in (32, 64, 128, 256):
        print(f"[parity] w4 M={m} k={k} exact", flush=True)
        assert_identical(gpu_run_t(xt, k, "exact"), oracle.exact(x, k), f"w4 M={m} k={k}")
    print(f"[parity] w4 M={m} k=256 uncapped", flush=True)
    assert_identical(gpu_run_t(xt, 256, "capped", -1, 0.0), oracle.exact(x, 256),
                     f"w4 M={m} uncapped")
    # Early-stopped search on tie-heavy rows: the staged first count often
    # jumps past its window here, so the search falls back to the row.
    for k in (32, 64, 128, 256):
        for mi, eps in ((2, 0.0), (4, 0.0), (6, 0.0), (-1, 0.01)):
            print(f"[parity] w4 M={m} k={k} capped max_iter={mi} eps={eps}", flush=True)
            assert_identical(gpu_run_t(xt, k, "capped", mi, eps), oracle.capped(x, k, mi, eps),
                             f"w4 M={m} k={k} capped {mi} {eps}")


def test_workload5_all_rows():
    """1,048,576 x 1,024 (4 GiB), every row checked, including the last rows
    (byte offsets beyond 2^32)."""
    x = workloads.config_input(5)
    xt = torch.from_numpy(x).to(dev())
    for mi in (2, 3, 4, 5, 6, 7, 8):
        print(f"[parity] w5 max_iter={mi}", flush=True)
        got = gpu_run_t(xt, 64, "capped", mi, 0.0)
        assert_identical(got, oracle.capped(x, 64, mi, 0.0), f"w5 max_iter={mi}")
        del got
    print("[parity] w5 exact", flush=True)
    assert_identical(gpu_run_t(xt, 64, "exact"), oracle.exact(x, 64), "w5 exact")
    del xt
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# Edge cases
# ---------------------------------------------------------------------------

ROW_LENGTHS = [1, 2, 5, 31, 63, 64, 65, 100, 127, 128, 129, 191, 192, 200, 255,
               256, 257, 300, 383, 384, 500, 512, 700, 1000, 1024, 1500, 2047,
               2048, 3000, 4095, 4096, 6000, 8191, 8192]


@pytest.mark.parametrize("m", ROW_LENGTHS)
def test_adversarial_rows(m):
    x = workloads.adversarial_rows(m)
    ks = sorted({k for k in (1, 2, m // 3, m - 1, m) if 1 <= k <= m})
    for k in ks:
        check(x, k, "exact", label=f"adv M={m}")
        if m <= 256:
            check(x, k, "exact", u8=True, label=f"adv M={m}")
        for mi, eps in ((-1, 0.0), (0, 0.0), (1, 0.0), (2, 0.0), (3, 0.0), (-1, 0.5), (6, 1e-3)):
            check(x, k, "capped", mi, eps, label=f"adv M={m}")
            if m <= 256 and mi in (-1, 2, 3):
                check(x, k, "capped", mi, eps, u8=True, label=f"adv M={m}")


# Value distributions away from the zero-centred normal rows the threshold
# model is tuned for: the first count then misses its window and the search
# retries with the row's mean and standard deviation, or falls back further
# (Newton steps, snaps, key bisection). The result must not change.
DISTRIBUTIONS = {
    "uniform01": lambda r, n, m: r.random((n, m)),
    "shift1000": lambda r, n, m: r.standard_normal((n, m)) + 1000.0,
    "negative": lambda r, n, m: -r.random((n, m)) - 5.0,
    "lognormal2": lambda r, n, m: np.exp(2.0 * r.standard_normal((n, m))),
    "relu": lambda r, n, m: np.maximum(r.standard_normal((n, m)), 0.0),
    "huge_offset": lambda r, n, m: r.standard_normal((n, m)) * 1e-3 + 3e30,
}


@pytest.mark.parametrize("dist", sorted(DISTRIBUTIONS))
@pytest.mark.parametrize("m,k", [(256, 32), (1000, 40), (4096, 64)])
def test_other_value_distributions(dist, m, k):
    rng = np.random.default_rng(900 + m)
    x = DISTRIBUTIONS[dist](rng, 1500, m).astype(np.float32) + np.float32(0.0)
    check(x, k, "exact", label=f"{dist} exact")
    check(x, k, "capped", 5, 0.0, label=f"{dist} capped")
    check(x, k, "capped", 2, 0.0, label=f"{dist} capped two steps")
    if m <= 256:
        check(x, k, "exact", u8=True, label=f"{dist} exact u8")


@pytest.mark.parametrize("n", [1, 2, 3, 5, 7, 1023, 4097, 30001])
def test_ragged_row_counts(n):
    m = 256 if n < 30000 else 100
    x = workloads.normal(n, m, seed=n)
    check(x, 7, "exact", label="ragged")
    check(x, 7, "capped", 4, 0.0, label="ragged")


def test_random_shapes_ties_and_scales():
    rng = np.random.default_rng(2024)
    for t in range(40):
        m = int(rng.integers(1, 1400))
        n = int(rng.integers(1, 300))
        k = int(rng.integers(1, m + 1))
        kind = t % 4
        if kind == 0:
            x = rng.standard_normal((n, m)).astype(np.float32)
        elif kind == 1:
            x = rng.integers(-3, 4, size=(n, m)).astype(np.float32)
        elif kind == 2:
            x = (rng.standard_normal((n, m)) * 10.0 ** rng.integers(-40, 37)).astype(np.float32)
        else:
            x = (rng.integers(-5, 6, size=(n, m)) * np.finfo(np.float32).smallest_subnormal).astype(np.float32)
        check(x, k, "exact", label=f"rand{t}")
        check(x, k, "capped", int(rng.integers(-1, 12)), float(rng.choice([0.0, 1e-3, 0.25])),
              label=f"rand{t}")
        if m <= 256:
            check(x, k, "exact", u8=True, label=f"rand{t} u8")


def test_random_long_rows():
    # Rows of 1,400 to 8,192 columns (16 to 128 slots per lane, full and
    # partial last slots, four-wave blocks), row counts spanning several
    # waves and a partial last block.
    rng = np.random.default_rng(77)
    for t in range(12):
        m = int(rng.integers(1400, 8193))
        n = int(rng.integers(1, 70))
        k = int(rng.integers(1, min(m, 512) + 1))
        if t % 3 == 0:
            x = rng.standard_normal((n, m)).astype(np.float32)
        elif t % 3 == 1:
            x = (np.round(rng.standard_normal((n, m)) * 4) / 4).astype(np.float32) + np.float32(0)
        else:
            x = (rng.standard_normal((n, m)) * 3 + 50).astype(np.float32)
        check(x, k, "exact", label=f"long{t}")
        check(x, k, "capped", int(rng.integers(-1, 10)), 0.0, label=f"long{t}")


# The capped search on rows held by four waves (more than 6,144 columns):
# ragged and full lengths, every branch of its tie fill (candidates only,
# wave 0's split fill, the staged fill over the row, and the full-row steps
# when the first count misses its window: shifted rows), with and without
# eps, and row counts above the resident grid.
@pytest.mark.parametrize("m", [6145, 7000, 8191, 8192])
def test_capped_long_rows_in_groups(m):
    rng = np.random.default_rng(900 + m)
    n = 3000 if m == 8192 else 700
    fams = {
        "normal": rng.standard_normal((n, m)).astype(np.float32),
        "ties": (np.round(rng.standard_normal((n, m)) * 4) / 4).astype(np.float32) + np.float32(0),
        "shifted": (rng.standard_normal((n, m)) * 3 + 50).astype(np.float32),
    }
    for name, x in fams.items():
        for k in (1, 32, 200):
            for it, eps in ((1, 0.0), (2, 0.0), (5, 0.0), (12, 0.0), (-1, 1e-3)):
                check(x, k, "capped", it, eps, label=f"group capped {name} M={m}")


def test_outputs_untouched_outside_bounds_and_deterministic():
    n, m, k = 777, 300, 40
    x = torch.from_numpy(workloads.normal(n, m, seed=5)).to(dev())
    guard = 4096
    vbuf = torch.full((n * k + 2 * guard,), 12345.0, dtype=torch.float32, device=dev())
    ibuf = torch.full((n * k + 2 * guard,), -777, dtype=torch.int32, device=dev())
    ov = vbuf[guard:guard + n * k].view(n, k)
    oi = ibuf[guard:guard + n * k].view(n, k)
    r = rt()
    r.rtopk_select_exact(x, k, out_val=ov, out_idx=oi)
    torch.cuda.synchronize()
    first = (ov.cpu().numpy().copy(), oi.cpu().numpy().copy())
    assert (vbuf[:guard] == 12345.0).all() and (vbuf[-guard:] == 12345.0).all()
    assert (ibuf[:guard] == -777).all() and (ibuf[-guard:] == -777).all()
    for _ in range(3):
        r.rtopk_select_exact(x, k, out_val=ov, out_idx=oi)
        torch.cuda.synchronize()
        assert (ov.cpu().numpy() == first[0]).all() and (oi.cpu().numpy() == first[1]).all()


def test_python_binding_errors_on_gpu():
    r = rt()
    x = torch.zeros((4, 300), dtype=torch.float32, device=dev())
    with pytest.raises(ValueError):
        r.rtopk_select(x, 0)
    with pytest.raises(ValueError):
        r.rtopk_select(x, 301)
    with pytest.raises(ValueError):
        r.rtopk_select(x, 3, eps=-1.0)
    with pytest.raises(NotImplementedError):
        r.rtopk_select_u8(x, 3)
    with pytest.raises(NotImplementedError):
        r.rtopk_select_exact(torch.zeros((2, 8193), device=dev()), 3)
    with pytest.raises(ValueError):
        r.rtopk_select(x.double(), 3)
    with pytest.raises(ValueError):
        r.rtopk_select(x.t(), 3)
    v, i = r.rtopk_select_exact(torch.zeros((0, 16), device=dev()), 3)
    assert v.shape == (0, 3) and i.shape == (0, 3)


def test_nonnull_stream():
    r = rt()
    x_np = workloads.normal(3000, 256, seed=9)
    x = torch.from_numpy(x_np).to(dev())
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        v, i = r.rtopk_select_exact(x, 32)
    s.synchronize()
    assert_identical((v.cpu().numpy(), i.cpu().numpy()), oracle.exact(x_np, 32), "stream")


# Short rows with few survivors take one lane per row (64 rows per wave), or
# four (16 rows per wave) for 65 to 128 columns keeping at most 16: row
# lengths around the 8/16/32/64/128-column classes, every survivor class,
# row counts that end inside a wave, tie-heavy and adversarial rows, and an
# input that starts one float past a 16-byte boundary (4-byte loads; the
# 65-128 column rows then take one wave per row).
@pytest.mark.parametrize("m", [1, 3, 8, 9, 16, 17, 31, 32, 33, 63, 64, 65, 68, 96, 100, 124,
                               127, 128])
def test_short_rows_many_per_wave(m):
    rng = np.random.default_rng(500 + m)
    for n in (1, 31, 32, 33, 63, 64, 65, 1000, 4097):
        for k in sorted({1, 2, 3, 5, 8, 9, 16} & set(range(1, m + 1))):
            fam = (n + k) % 3
            if fam == 0:
                x = rng.standard_normal((n, m)).astype(np.float32)
            elif fam == 1:
                x = rng.integers(-2, 3, size=(n, m)).astype(np.float32)
            else:
                x = np.tile(workloads.adversarial_rows(m), (n // 16 + 1, 1))[:n]
            x = np.ascontiguousarray(x) + np.float32(0.0)
            check(x, k, "exact", label=f"short M={m} n={n}")
            check(x, k, "exact", u8=True, label=f"short M={m} n={n}")
            if n == 1000:
                check(x, k, "capped", -1, 0.0, label=f"short uncapped M={m}")
    # Misaligned start: a view one float into a padded buffer.
    x = workloads.normal(777, m, seed=m)
    buf = torch.zeros(777 * m + 1, dtype=torch.float32, device=dev())
    buf[1:].copy_(torch.from_numpy(x.reshape(-1)))
    xt = buf[1:].view(777, m)
    for k in sorted({1, 4, 8, 16} & set(range(1, m + 1))):
        assert_identical(gpu_run_t(xt, k, "exact"), oracle.exact(x, k), f"short misaligned M={m}")


# Batches larger than one resident grid: each wave of the staged lane kernel
# loops over several groups of 64 rows, loading the next group while it
# selects the current one; the row counts end inside a group. Normal and
# tie-heavy rows (quarter steps, about 30 distinct values).
@pytest.mark.parametrize("n,m,k", [(2097152 + 5, 32, 4), (1048576 + 37, 64, 8),
                                   (600001, 48, 6), (700003, 20, 3), (500009, 64, 1),
                                   (1048576 + 17, 128, 16), (600011, 100, 12),
                                   (500009, 68, 5)])
def test_short_rows_beyond_resident_grid(n, m, k):
    x = workloads.normal(n, m, seed=n % 1000)
    check(x, k, "exact", u8=True, label=f"short n={n} M={m}")
    xq = np.round(x[: n // 2] * 4) / 4 + np.float32(0.0)
    check(np.ascontiguousarray(xq.astype(np.float32)), k, "exact",
          label=f"short ties n={n // 2} M={m}")


# Rows of 257 to 384 columns (six slots per lane, groups of four rows per
# wave): normal rows take the candidate window, shifted and uniform ones the
# fallback; row counts that end inside a group leave rows of it unused.
@pytest.mark.parametrize("m", [257, 320, 383, 384])
def test_six_slot_rows(m):
    rng = np.random.default_rng(1300 + m)
    for n in (1, 2, 3, 5, 6, 7, 4099):
        x = workloads.normal(n, m, seed=1300 + n)
        for k in (1, 16, 32, 64, m // 2):
            check(x, k, "exact", label=f"six-slot M={m} n={n} k={k}")
    x = (rng.standard_normal((777, m)) + 1000.0).astype(np.float32)
    check(x, 32, "exact", label=f"six-slot shifted M={m}")
    x = rng.random((777, m)).astype(np.float32)
    check(x, 24, "exact", label=f"six-slot uniform M={m}")
    x = workloads.grid_ties(555, m, 5)
    check(x, 40, "exact", label=f"six-slot ties M={m}")
