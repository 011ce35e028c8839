"""GPU parity of the MaxK nonlinearity against the oracle, bit for bit:
the backward scatter (rtopk_maxk_backward[_u8]) and the forward
(rtopk_maxk_forward[_u8]: dense output plus the compressed pair).

Neither does arithmetic on the values it moves: every dense element is the
bits of one input element or +0.0, so the bar is identity with
oracle.maxk_backward (on rows whose indices are distinct) and with
oracle.maxk_forward. Backward index sets come from the oracle's exact top-k of
seeded workload rows (ascending, as the forward pass produces them) and from
seeded random permutations (unsorted), with out-of-range entries mixed in
where the index type allows them. Shapes cover every kernel path (the
one-pass and chunked scatters, the fused forward up to 1024 columns and the
two-launch forward beyond), 16-byte and 4-byte stores (M % 4, misaligned
outputs), adversarial rows (ties, +-0, subnormals, +-FLT_MAX), ragged row
counts and the full 262,144 x 256 headline shape.
"""

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def dev():
    return torch.device("cuda:0")


def rt():
    import row_wise_top_amd
    return row_wise_top_amd


def random_indices(rng, n, m, k):
    """Distinct, unsorted column indices per row."""
    return np.stack([rng.permutation(m)[:k] for _ in range(n)]).astype(np.int32)


def gpu_backward(g, idx, m, u8=False, out=None, stream=None):
    gt = torch.from_numpy(np.ascontiguousarray(g)).to(dev())
    it = torch.from_numpy(np.ascontiguousarray(idx.astype(np.uint8 if u8 else np.int32))).to(dev())
    res = rt().rtopk_maxk_backward(gt, it, m, grad_x=out, stream=stream)
    torch.cuda.synchronize()
    return res.cpu().numpy()


def assert_bits_equal(got, want, label):
    bad = np.flatnonzero((got.view(np.uint32) != want.view(np.uint32)).any(axis=1))
    assert bad.size == 0, f"{label}: {bad.size} rows differ, first row {bad[0]}"


SHAPES = [  # (n, m, k)
    (1, 1, 1), (7, 5, 3), (33, 63, 10), (64, 64, 64), (300, 100, 32),
    (257, 255, 17), (300, 256, 32), (129, 257, 100), (100, 511, 256),
    (50, 1000, 257), (70, 1024, 64), (40, 1025, 31), (30, 3000, 700),
    (9, 8192, 8192), (20, 8192, 40),
]


@pytest.mark.parametrize("n,m,k", SHAPES)
def test_backward_random_indices(n, m, k):
    rng = np.random.default_rng(1000 + m + k)
    g = rng.standard_normal((n, k)).astype(np.float32)
    idx = random_indices(rng, n, m, k)
    assert_bits_equal(gpu_backward(g, idx, m), oracle.maxk_backward(g, idx, m),
                      f"int32 n={n} m={m} k={k}")
    if m <= 256:
        assert_bits_equal(gpu_backward(g, idx, m, u8=True),
                          oracle.maxk_backward(g, idx, m), f"u8 n={n} m={m} k={k}")


@pytest.mark.parametrize("cfg", [1, 3])
def test_backward_of_forward_indices(cfg):
    # The index sets MaxK's forward pass produces: exact top-k of workload rows.
    n = 4096
    x = workloads.config_input(cfg, n, 256)
    _, idx = oracle.exact(x, 32)
    rng = np.random.default_rng(40 + cfg)
    g = rng.standard_normal((n, 32)).astype(np.float32)
    want = oracle.maxk_backward(g, idx, 256)
    assert_bits_equal(gpu_backward(g, idx, 256), want, f"cfg{cfg} int32")
    assert_bits_equal(gpu_backward(g, idx, 256, u8=True), want, f"cfg{cfg} u8")


def test_compressed_rows_back_to_dense_maxk():
    # Scattering the survivors (sp_data, sp_index) gives the dense MaxK output.
    x = workloads.config_input(3, 2048, 256)
    y, vals, idx = oracle.maxk_forward(x, 32)
    assert_bits_equal(gpu_backward(vals, idx, 256, u8=True), y, "dense from compressed")


def test_out_of_range_entries_are_ignored():
    rng = np.random.default_rng(51)
    n, m, k = 200, 100, 20
    g = rng.standard_normal((n, k)).astype(np.float32)
    idx = random_indices(rng, n, m, k)
    idx[::3, 0] = -1
    idx[1::3, 5] = m
    idx[2::3, 7] = 2**30
    assert_bits_equal(gpu_backward(g, idx, m), oracle.maxk_backward(g, idx, m), "int32 oob")
    idx8 = random_indices(rng, n, m, k)
    idx8[::2, 3] = 200  # a byte index past M = 100
    assert_bits_equal(gpu_backward(g, idx8, m, u8=True),
                      oracle.maxk_backward(g, idx8, m), "u8 oob")


@pytest.mark.parametrize("m", [256, 2048])
def test_misaligned_output_and_guard_bands(m):
    # The output starts 4 bytes past a 16-byte boundary (the kernel must use
    # 4-byte stores) and sits between guard bands that must stay untouched.
    rng = np.random.default_rng(60 + m)
    n, k = 123, 32
    g = rng.standard_normal((n, k)).astype(np.float32)
    idx = random_indices(rng, n, m, k)
    guard = 4096
    buf = torch.full((n * m + 2 * guard + 1,), 7.0, dtype=torch.float32, device=dev())
    out = buf[guard + 1: guard + 1 + n * m].view(n, m)
    assert out.data_ptr() % 16 == 4
    got = gpu_backward(g, idx, m, out=out)
    assert_bits_equal(got, oracle.maxk_backward(g, idx, m), f"misaligned m={m}")
    host = buf.cpu().numpy()
    assert np.all(host[:guard + 1] == 7.0) and np.all(host[guard + 1 + n * m:] == 7.0)


def test_ragged_row_counts_and_stream():
    rng = np.random.default_rng(70)
    m, k = 256, 32
    s = torch.cuda.Stream(device=dev())
    for n in (1, 2, 3, 5, 1023, 1025, 4097):
        g = rng.standard_normal((n, k)).astype(np.float32)
        idx = random_indices(rng, n, m, k)
        with torch.cuda.stream(s):
            got = gpu_backward(g, idx, m, u8=True, stream=s)
        assert_bits_equal(got, oracle.maxk_backward(g, idx, m), f"n={n}")


def test_full_headline_shape():
    n, m, k = 262144, 256, 32
    x = workloads.config_input(3, n, m)
    _, idx = oracle.exact(x, k)
    rng = np.random.default_rng(80)
    g = rng.standard_normal((n, k)).astype(np.float32)
    assert_bits_equal(gpu_backward(g, idx, m, u8=True), oracle.maxk_backward(g, idx, m),
                      "262144 x 256 u8")


# --------------------------------------------------------------------------
# MaxK forward (rtopk_maxk_forward[_u8]): dense output plus compressed pair.
# --------------------------------------------------------------------------

def gpu_forward(x_np, k, u8=False, y=None):
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to(dev())
    yy, v, i = rt().rtopk_maxk_forward(x, k, y=y, index_dtype=torch.uint8 if u8 else None)
    torch.cuda.synchronize()
    return yy.cpu().numpy(), v.cpu().numpy(), i.cpu().numpy().astype(np.int32)


def assert_forward_equal(got, want, label):
    gy, gv, gi = got
    wy, wv, wi = want
    assert_bits_equal(gy, wy, label + " y")
    assert_bits_equal(gv, wv, label + " sp_data")
    bad = np.flatnonzero((gi != wi).any(axis=1))
    assert bad.size == 0, f"{label} sp_index: {bad.size} rows differ, first {bad[0]}"


FORWARD_SHAPES = [  # (n, m, k): every slot bucket; fused up to 1024, two launches beyond
    (5, 1, 1), (33, 5, 2), (64, 63, 7), (100, 64, 32), (129, 100, 10), (77, 200, 64),
    (300, 255, 32), (1000, 256, 32), (70, 256, 256), (257, 257, 32), (60, 300, 150),
    (50, 500, 16), (40, 512, 100), (30, 700, 64), (20, 1000, 500), (65, 1024, 64),
    (20, 1025, 32), (16, 2048, 64), (8, 5000, 2500), (6, 8192, 256),
]


@pytest.mark.parametrize("n,m,k", FORWARD_SHAPES)
@pytest.mark.parametrize("data", ["normal", "maxk", "grid"])
def test_forward_shapes(n, m, k, data):
    if data == "normal":
        x = workloads.normal(n, m, 300 + m)
    elif data == "maxk":
        x = workloads.maxk_activation(n, m, workloads.CONFIG_SEEDS[3])
    else:
        x = workloads.grid_ties(n, m, 5)
    want = oracle.maxk_forward(x, k)
    assert_forward_equal(gpu_forward(x, k), want, f"i32 {data} n={n} m={m} k={k}")
    if m <= 256:
        assert_forward_equal(gpu_forward(x, k, u8=True), want, f"u8 {data} n={n} m={m} k={k}")


@pytest.mark.parametrize("m", [1, 3, 64, 100, 256, 1000, 1024, 2000])
def test_forward_adversarial_rows(m):
    x = workloads.adversarial_rows(m)
    for k in sorted({1, max(1, m // 3), max(1, m - 1), m}):
        assert_forward_equal(gpu_forward(x, k), oracle.maxk_forward(x, k),
                             f"adversarial m={m} k={k}")


@pytest.mark.parametrize("m", [256, 2048])
def test_forward_misaligned_dense_output(m):
    n, k = 150, 32
    x = workloads.normal(n, m, 400 + m)
    guard = 4096
    buf = torch.full((n * m + 2 * guard + 1,), 7.0, dtype=torch.float32, device=dev())
    y = buf[guard + 1: guard + 1 + n * m].view(n, m)
    assert y.data_ptr() % 16 == 4
    got = gpu_forward(x, k, y=y)
    assert_forward_equal(got, oracle.maxk_forward(x, k), f"misaligned m={m}")
    host = buf.cpu().numpy()
    assert np.all(host[:guard + 1] == 7.0) and np.all(host[guard + 1 + n * m:] == 7.0)


def test_forward_then_backward_round_trip():
    # Backward of the forward's survivors with the survivors as gradient
    # reproduces the dense forward output.
    x = workloads.config_input(3, 8192, 256)
    y, v, i = gpu_forward(x, 32, u8=True)
    back = gpu_backward(v, i, 256, u8=True)
    assert_bits_equal(back, y, "round trip")


def test_forward_full_headline_shape():
    n, m, k = 262144, 256, 32
    x = workloads.config_input(3, n, m)
    assert_forward_equal(gpu_forward(x, k, u8=True), oracle.maxk_forward(x, k),
                         "262144 x 256 u8")
