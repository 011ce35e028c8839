"""The C ABI (include/rtopk.h): symbols, status strings and host-side
validation. Runs without a GPU: every call here is rejected (or is the N = 0
no-op) before the library touches the HIP runtime."""

import ctypes
import os
import re

import pytest

import row_wise_top_amd as rt
from row_wise_top_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "rtopk.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rtopk_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted([
        "rtopk_select", "rtopk_select_exact", "rtopk_select_u8",
        "rtopk_select_exact_u8", "rtopk_select_bucketed", "rtopk_select_bucketed_u8",
        "rtopk_maxk_forward", "rtopk_maxk_forward_u8",
        "rtopk_maxk_backward", "rtopk_maxk_backward_u8", "rtopk_cbsr_spgemm",
        "rtopk_cbsr_spgemm_u8", "rtopk_cbsr_sspmm", "rtopk_cbsr_sspmm_u8",
        "rtopk_status_string"])


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code in range(4):
        s = rt.rtopk_status_string(code)
        assert isinstance(s, str) and s
    assert rt.rtopk_status_string(0) == "success"
    assert rt.rtopk_status_string(99) == "unknown status"


def call(fn, *args):
    return getattr(rt.lib(), fn)(*args)


CAPPED = ["rtopk_select", "rtopk_select_u8"]
EXACT = ["rtopk_select_exact", "rtopk_select_exact_u8"]
FAKE = 0x1000  # never dereferenced: every case below fails validation first


@pytest.mark.parametrize("fn", CAPPED + EXACT)
def test_n_zero_is_a_noop(fn):
    if fn in CAPPED:
        assert call(fn, None, 0, 16, 4, -1, 0.0, None, None, None) == 0
    else:
        assert call(fn, None, 0, 16, 4, None, None, None) == 0


@pytest.mark.parametrize("fn", CAPPED + EXACT)
@pytest.mark.parametrize("n,m,k,code", [
    (-1, 16, 4, 1),      # N < 0
    (4, 0, 1, 1),        # M < 1
    (4, 16, 0, 1),       # k < 1
    (4, 16, 17, 1),      # k > M
    (4, 8193, 4, 2),     # M above the supported maximum
])
def test_shape_errors(fn, n, m, k, code):
    if fn in CAPPED:
        rc = call(fn, FAKE, n, m, k, -1, 0.0, FAKE, FAKE, None)
    else:
        rc = call(fn, FAKE, n, m, k, FAKE, FAKE, None)
    assert rc == code


@pytest.mark.parametrize("fn", ["rtopk_select_u8", "rtopk_select_exact_u8"])
def test_u8_requires_short_rows(fn):
    if fn in CAPPED:
        assert call(fn, FAKE, 4, 257, 4, -1, 0.0, FAKE, FAKE, None) == 2
    else:
        assert call(fn, FAKE, 4, 257, 4, FAKE, FAKE, None) == 2


@pytest.mark.parametrize("fn", CAPPED)
@pytest.mark.parametrize("eps", [-1.0, float("nan"), -1e-30])
def test_bad_eps(fn, eps):
    assert call(fn, FAKE, 4, 16, 4, -1, eps, FAKE, FAKE, None) == 1


@pytest.mark.parametrize("fn", CAPPED + EXACT)
@pytest.mark.parametrize("which", [0, 1, 2])
def test_null_pointers(fn, which):
    ptrs = [FAKE, FAKE, FAKE]
    ptrs[which] = None
    if fn in CAPPED:
        rc = call(fn, ptrs[0], 4, 16, 4, -1, 0.0, ptrs[1], ptrs[2], None)
    else:
        rc = call(fn, ptrs[0], 4, 16, 4, ptrs[1], ptrs[2], None)
    assert rc == 1


BACKWARD = ["rtopk_maxk_backward", "rtopk_maxk_backward_u8"]


@pytest.mark.parametrize("fn", BACKWARD)
def test_backward_n_zero_is_a_noop(fn):
    assert call(fn, None, None, 0, 16, 4, None, None) == 0


@pytest.mark.parametrize("fn", BACKWARD)
@pytest.mark.parametrize("n,m,k,code", [
    (-1, 16, 4, 1),      # N < 0
    (4, 0, 1, 1),        # M < 1
    (4, 16, 0, 1),       # k < 1
    (4, 16, 17, 1),      # k > M
    (4, 8193, 4, 2),     # M above the supported maximum
])
def test_backward_shape_errors(fn, n, m, k, code):
    assert call(fn, FAKE, FAKE, n, m, k, FAKE, None) == code


def test_backward_u8_requires_short_rows():
    assert call("rtopk_maxk_backward_u8", FAKE, FAKE, 4, 257, 4, FAKE, None) == 2


@pytest.mark.parametrize("fn", BACKWARD)
@pytest.mark.parametrize("which", [0, 1, 2])
def test_backward_null_pointers(fn, which):
    ptrs = [FAKE, FAKE, FAKE]
    ptrs[which] = None
    assert call(fn, ptrs[0], ptrs[1], 4, 16, 4, ptrs[2], None) == 1


FORWARD = ["rtopk_maxk_forward", "rtopk_maxk_forward_u8"]


@pytest.mark.parametrize("fn", FORWARD)
def test_forward_n_zero_is_a_noop(fn):
    assert call(fn, None, 0, 16, 4, None, None, None, None) == 0


@pytest.mark.parametrize("fn", FORWARD)
@pytest.mark.parametrize("n,m,k,code", [
    (-1, 16, 4, 1), (4, 0, 1, 1), (4, 16, 0, 1), (4, 16, 17, 1), (4, 8193, 4, 2),
])
def test_forward_shape_errors(fn, n, m, k, code):
    assert call(fn, FAKE, n, m, k, FAKE, FAKE, FAKE, None) == code


def test_forward_u8_requires_short_rows():
    assert call("rtopk_maxk_forward_u8", FAKE, 4, 257, 4, FAKE, FAKE, FAKE, None) == 2


@pytest.mark.parametrize("fn", FORWARD)
@pytest.mark.parametrize("which", [0, 1, 2, 3])
def test_forward_null_pointers(fn, which):
    ptrs = [FAKE, FAKE, FAKE, FAKE]
    ptrs[which] = None
    assert call(fn, ptrs[0], 4, 16, 4, ptrs[1], ptrs[2], ptrs[3], None) == 1


BUCKETED = ["rtopk_select_bucketed", "rtopk_select_bucketed_u8"]


@pytest.mark.parametrize("fn", BUCKETED)
def test_bucketed_n_zero_is_a_noop(fn):
    assert call(fn, None, 0, 16, 4, 2, None, None, None) == 0


@pytest.mark.parametrize("fn", BUCKETED)
@pytest.mark.parametrize("n,m,k,b,code", [
    (-1, 16, 4, 2, 1),      # N < 0
    (4, 16, 17, 1, 1),      # k > M
    (4, 16, 4, 0, 1),       # no buckets
    (4, 16, 4, 3, 1),       # 3 does not divide M
    (4, 18, 4, 3, 1),       # 3 does not divide k
    (4, 8193, 4, 1, 2),     # M above the maximum
])
def test_bucketed_argument_errors(fn, n, m, k, b, code):
    assert call(fn, FAKE, n, m, k, b, FAKE, FAKE, None) == code


def test_bucketed_long_buckets_not_supported():
    assert call("rtopk_select_bucketed", FAKE, 4, 2048, 8, 1, FAKE, FAKE, None) == 2
    assert call("rtopk_select_bucketed_u8", FAKE, 4, 512, 8, 2, FAKE, FAKE, None) == 2


@pytest.mark.parametrize("fn", BUCKETED)
@pytest.mark.parametrize("which", [0, 1, 2])
def test_bucketed_null_pointers(fn, which):
    ptrs = [FAKE, FAKE, FAKE]
    ptrs[which] = None
    assert call(fn, ptrs[0], 4, 16, 4, 2, ptrs[1], ptrs[2], None) == 1


SPGEMM = ["rtopk_cbsr_spgemm", "rtopk_cbsr_spgemm_u8"]


@pytest.mark.parametrize("fn", SPGEMM)
def test_spgemm_no_rows_is_a_noop(fn):
    assert call(fn, None, None, None, 0, 0, 0, None, None, 16, 4, None, None) == 0


@pytest.mark.parametrize("fn", SPGEMM)
@pytest.mark.parametrize("n_dst,n_src,nnz,m,k,code", [
    (-1, 4, 4, 16, 4, 1),     # n_dst < 0
    (4, -1, 4, 16, 4, 1),     # n_src < 0
    (4, 4, -1, 16, 4, 1),     # nnz < 0
    (4, 0, 4, 16, 4, 1),      # edges but no source rows
    (4, 4, 4, 16, 17, 1),     # k > M
    (4, 4, 4, 0, 1, 1),       # M < 1
    (4, 4, 4, 8193, 4, 2),    # M above the maximum
])
def test_spgemm_argument_errors(fn, n_dst, n_src, nnz, m, k, code):
    assert call(fn, FAKE, FAKE, FAKE, n_dst, n_src, nnz, FAKE, FAKE, m, k, FAKE, None) == code


def test_spgemm_u8_requires_short_rows():
    assert call("rtopk_cbsr_spgemm_u8", FAKE, FAKE, FAKE, 4, 4, 4, FAKE, FAKE, 257, 4,
                FAKE, None) == 2


@pytest.mark.parametrize("fn", SPGEMM)
@pytest.mark.parametrize("which", [0, 1, 2, 3, 4, 5])
def test_spgemm_null_pointers(fn, which):
    ptrs = [FAKE] * 6
    ptrs[which] = None
    assert call(fn, ptrs[0], ptrs[1], ptrs[2], 4, 4, 4, ptrs[3], ptrs[4], 16, 4,
                ptrs[5], None) == 1


SSPMM = ["rtopk_cbsr_sspmm", "rtopk_cbsr_sspmm_u8"]


@pytest.mark.parametrize("fn", SSPMM)
def test_sspmm_no_source_rows_is_a_noop(fn):
    assert call(fn, None, None, None, 4, 0, 0, None, None, 16, 4, None, None) == 0


@pytest.mark.parametrize("fn", SSPMM)
@pytest.mark.parametrize("n_dst,n_src,nnz,m,k,code", [
    (-1, 4, 4, 16, 4, 1), (4, -1, 4, 16, 4, 1), (4, 4, -1, 16, 4, 1),
    (4, 0, 4, 16, 4, 1), (4, 4, 4, 16, 17, 1), (4, 4, 4, 8193, 4, 2),
])
def test_sspmm_argument_errors(fn, n_dst, n_src, nnz, m, k, code):
    assert call(fn, FAKE, FAKE, FAKE, n_dst, n_src, nnz, FAKE, FAKE, m, k, FAKE, None) == code


@pytest.mark.parametrize("fn", SSPMM)
@pytest.mark.parametrize("which", [0, 1, 2, 3, 4, 5])
def test_sspmm_null_pointers(fn, which):
    ptrs = [FAKE] * 6
    ptrs[which] = None
    assert call(fn, ptrs[0], ptrs[1], ptrs[2], 4, 4, 4, ptrs[3], ptrs[4], 16, 4,
                ptrs[5], None) == 1


def _no_device() -> bool:
    # Counting devices does not initialise the GPU on this image.
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


# Fully valid calls, each the first (or only) launch of its entry point. With
# no device visible the launch itself fails: the call must report
# RTOPK_ERROR_LAUNCH (and, for the two-kernel calls, stop before the second
# launch). Never run where a GPU is visible: the pointers are not real.
LAUNCH_CASES = [
    ("rtopk_select", (FAKE, 4, 16, 4, 2, 0.0, FAKE, FAKE, None)),
    ("rtopk_select_u8", (FAKE, 4, 16, 4, -1, 0.0, FAKE, FAKE, None)),
    ("rtopk_select_exact", (FAKE, 4, 16, 4, FAKE, FAKE, None)),
    ("rtopk_select_exact_u8", (FAKE, 4, 16, 4, FAKE, FAKE, None)),
    ("rtopk_select_bucketed", (FAKE, 4, 16, 4, 2, FAKE, FAKE, None)),
    ("rtopk_maxk_forward", (FAKE, 4, 16, 4, FAKE, FAKE, FAKE, None)),
    ("rtopk_maxk_forward", (FAKE, 4, 2048, 4, FAKE, FAKE, FAKE, None)),  # two kernels
    ("rtopk_maxk_backward", (FAKE, FAKE, 4, 16, 4, FAKE, None)),
    ("rtopk_cbsr_spgemm", (FAKE, FAKE, FAKE, 4, 4, 600, FAKE, FAKE, 16, 4, FAKE, None)),
    ("rtopk_cbsr_sspmm", (FAKE, FAKE, FAKE, 4, 4, 600, FAKE, FAKE, 16, 4, FAKE, None)),
]


@pytest.mark.skipif(not _no_device(), reason="needs a host with no GPU visible")
@pytest.mark.parametrize("fn,args", LAUNCH_CASES, ids=[c[0] for c in LAUNCH_CASES])
def test_launch_failure_maps_to_launch_status(fn, args):
    assert call(fn, *args) == 3
