"""GPU parity of the bucketed approximate top-k (rtopk_select_bucketed[_u8])
against oracle.bucketed, bit for bit: the same columns (relative to the whole
row, bucket by bucket) and the same value bits. Bucket lengths cover every
slot bucket of the kernels up to 1024, ragged bucket lengths, ties and the
full 262,144 x 256 shape with 8 buckets."""

import numpy as np
import pytest

import oracle
import workloads

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def gpu_bucketed(x_np, k, b, u8=False):
    import row_wise_top_amd as rt
    x = torch.from_numpy(np.ascontiguousarray(x_np)).to("cuda:0")
    v, i = rt.rtopk_select_bucketed(x, k, b, index_dtype=torch.uint8 if u8 else None)
    torch.cuda.synchronize()
    return v.cpu().numpy(), i.cpu().numpy().astype(np.int32)


def assert_identical(got, want, label):
    gv, gi = got
    wv, wi = want
    bad = np.flatnonzero((gi != wi).any(axis=1) |
                         (gv.view(np.uint32) != wv.view(np.uint32)).any(axis=1))
    assert bad.size == 0, f"{label}: {bad.size} rows differ, first {bad[0]}"


CASES = [  # (n, m, k, buckets)
    (100, 8, 4, 2), (257, 64, 8, 2), (300, 100, 20, 5), (129, 256, 32, 8),
    (500, 256, 32, 4), (77, 256, 64, 2), (64, 256, 256, 256), (99, 256, 16, 16),
    (60, 384, 24, 3), (50, 1000, 40, 4), (40, 1024, 64, 1), (33, 2048, 64, 2),
    (20, 3072, 48, 3), (17, 8192, 64, 8), (9, 8192, 512, 8),
    # Buckets of at most 64 columns keeping at most 8 (one lane per bucket):
    # every width class (8, 16, 32, 64) and survivor class (1, 2, 4, 8),
    # widths that are not multiples of 4, and survivors short of the class.
    (203, 12, 4, 4), (203, 12, 8, 4), (203, 12, 12, 4), (150, 40, 40, 8),
    (150, 56, 56, 8), (97, 52, 24, 4), (97, 62, 16, 2), (300, 256, 64, 8),
    (81, 96, 12, 4), (70, 2048, 512, 64), (66, 8192, 256, 256),
    (120, 256, 32, 4), (90, 200, 20, 4), (77, 96, 8, 2), (60, 128, 2, 2),
    (45, 132, 24, 3),
    # Buckets of 65 to 128 columns keeping at most 16 (four lanes per bucket,
    # 16 buckets per wave) where the width is a multiple of 4; other widths
    # take the wave kernel.
    (257, 256, 32, 2), (300, 200, 10, 2), (130, 272, 24, 4), (99, 340, 20, 4),
    (65, 384, 12, 3), (70, 248, 2, 2), (1000, 256, 16, 2), (31, 256, 30, 2),
    (33, 136, 32, 2), (47, 512, 64, 4),
    # Buckets of 257 to 384 columns: the wave kernel, groups of four rows.
    (37, 768, 64, 2), (41, 640, 20, 2), (5, 1152, 60, 3),
]


@pytest.mark.parametrize("n,m,k,b", CASES)
@pytest.mark.parametrize("data", ["normal", "maxk", "grid"])
def test_bucketed_matches_oracle(n, m, k, b, data):
    if data == "normal":
        x = workloads.normal(n, m, 500 + m + b)
    elif data == "maxk":
        x = workloads.maxk_activation(n, m, workloads.CONFIG_SEEDS[3])
    else:
        x = workloads.grid_ties(n, m, 5)
    want = oracle.bucketed(x, k, b)
    assert_identical(gpu_bucketed(x, k, b), want, f"i32 {data} n={n} m={m} k={k} b={b}")
    if m <= 256:
        assert_identical(gpu_bucketed(x, k, b, u8=True), want, f"u8 {data} n={n} m={m} k={k} b={b}")


@pytest.mark.parametrize("m,b", [(6, 3), (100, 4), (256, 8), (1024, 2)])
def test_bucketed_adversarial_rows(m, b):
    x = workloads.adversarial_rows(m)
    for k in sorted({b, 2 * b if 2 * b <= m else b, m}):
        if k % b:
            continue
        assert_identical(gpu_bucketed(x, k, b), oracle.bucketed(x, k, b),
                         f"adversarial m={m} b={b} k={k}")


def test_bucketed_ragged_row_counts():
    for n in (1, 2, 3, 5, 17, 1023, 1025):
        x = workloads.normal(n, 256, 600 + n)
        assert_identical(gpu_bucketed(x, 32, 8, u8=True), oracle.bucketed(x, 32, 8), f"n={n}")


@pytest.mark.parametrize("b", [8, 4, 2])
def test_bucketed_full_shape(b):
    x = workloads.config_input(3, 262144, 256)
    assert_identical(gpu_bucketed(x, 32, b, u8=True), oracle.bucketed(x, 32, b),
                     f"262144 x 256 k=32 b={b}")


@pytest.mark.parametrize("m,k,b", [(256, 32, 8), (96, 12, 4), (64, 16, 16), (256, 32, 4),
                                   (256, 32, 2)])
def test_bucketed_unaligned_input(m, k, b):
    # A matrix starting one float past a 16-byte boundary: the short-bucket
    # kernel then reads with 4-byte loads.
    import row_wise_top_amd as rt
    n = 211
    x_np = workloads.normal(n, m, 700 + m)
    flat = torch.zeros(n * m + 1, dtype=torch.float32, device="cuda:0")
    x = flat[1:].view(n, m)
    x.copy_(torch.from_numpy(x_np).to("cuda:0"))
    assert x.data_ptr() % 16 != 0
    v, i = rt.rtopk_select_bucketed(x, k, b)
    torch.cuda.synchronize()
    assert_identical((v.cpu().numpy(), i.cpu().numpy().astype(np.int32)),
                     oracle.bucketed(x_np, k, b), f"unaligned m={m} k={k} b={b}")


@pytest.mark.parametrize("m,k,b", [(256, 32, 8), (256, 16, 8), (128, 16, 8), (96, 12, 4),
                                   (256, 32, 2), (256, 30, 2), (200, 20, 2)])
@pytest.mark.parametrize("u8", [False, True])
def test_bucketed_unaligned_outputs(m, k, b, u8):
    # Outputs starting one element past a 16-byte boundary: the short-bucket
    # kernels then store entry by entry instead of in 16-byte pieces.
    import row_wise_top_amd as rt
    n = 203
    x_np = workloads.normal(n, m, 800 + m + k)
    x = torch.from_numpy(x_np).to("cuda:0")
    dt = torch.uint8 if u8 else torch.int32
    fv = torch.full((n * k + 1,), -1.0, dtype=torch.float32, device="cuda:0")
    fi = torch.zeros((n * k + 1,), dtype=dt, device="cuda:0")
    v, i = fv[1:].view(n, k), fi[1:].view(n, k)
    assert v.data_ptr() % 16 != 0 and i.data_ptr() % 16 != 0
    rt.rtopk_select_bucketed(x, k, b, out_val=v, out_idx=i, index_dtype=dt)
    torch.cuda.synchronize()
    assert fv[0].item() == -1.0 and fi[0].item() == 0
    assert_identical((v.cpu().numpy(), i.cpu().numpy().astype(np.int32)),
                     oracle.bucketed(x_np, k, b), f"unaligned outputs m={m} k={k} b={b} u8={u8}")


def survivor_layout_rows(n, m, seed, layouts=(0, 1, 2)):
    """Rows of 128-column buckets whose largest places sit in one quarter
    (layout 0: one lane of the four-lane kernel keeps them all), four to a
    quarter (1), or are all equal (2: the lowest columns, hence the first
    quarter, keep them); the given layouts take turns over the buckets, so
    that with several one wave of 16 buckets mixes them."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, m)).astype(np.float32)
    for r in range(n):
        for j in range(m // 128):
            bkt = x[r, 128 * j:128 * (j + 1)]
            layout = layouts[(r * (m // 128) + j) % len(layouts)]
            if layout == 0:
                q = (r + j) % 4
                bkt[32 * q:32 * q + 32] += np.float32(100.0)
            elif layout == 1:
                for q in range(4):
                    bkt[32 * q + rng.choice(32, 4, replace=False)] += np.float32(100.0)
            else:
                bkt[:] = np.float32(1.5)
    return x


@pytest.mark.parametrize("layouts", [(0, 1, 2), (1,), (0,), (2,), (1,) * 47 + (0,)])
@pytest.mark.parametrize("k", [8, 16, 24, 32])
def test_four_lane_survivor_layouts(k, layouts):
    # 2 buckets of 128 keeping k / 2 each: the four-lane kernel, whose lanes
    # run their survivor slots in chunks of four and skip the chunks that no
    # lane of the wave needs (all of a bucket's survivors in one lane needs
    # every chunk; four to a quarter in every bucket of a wave only the
    # first; one one-quarter bucket in 48 makes every third wave of 16
    # buckets need them all again).
    x = survivor_layout_rows(1001, 256, 17, layouts)
    want = oracle.bucketed(x, k, 2)
    assert_identical(gpu_bucketed(x, k, 2), want, f"layouts {layouts} i32 k={k}")
    assert_identical(gpu_bucketed(x, k, 2, u8=True), want, f"layouts {layouts} u8 k={k}")
