"""CPU oracle for row-wise top-k selection -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the CPU-baseline leg of ``bench.py``
may import this package. The GPU library never does, and nothing here is
shared with it: the oracle is a separate C++ file (``rtopk_oracle.cpp``)
compiled with g++ and loaded through ctypes.

``exact`` is the plain definition of row-wise top-k (RTop-K summary page,
"Problem"/"Approach"; MaxK-GNN review, "How MaxK-GNN works": exactly k
survivors per row), ties at the k-th value going to the lowest indices, by
partial selection (``std::nth_element``); ``exact_by_sort`` reaches the same
result through a full stable sort.
``capped`` is the threshold search with early stopping and tie fill of the RTop-K
summary page, "Approach", in the reading spelled out in ``rtopk_oracle.cpp``.
Both return the survivors of each row in ascending index order.
``bucketed`` is the bucketed approximate top-k (page "Approximate Top-k for
Increased Parallelism"): exact top-(k/b) of each of b contiguous buckets.
``spgemm`` is MaxK-GNN's forward aggregation Y = A X (CSR graph A, X given
by its compressed MaxK rows), summed in double and rounded once.
``sspmm`` is its backward to the compressed features: (A^T dY) sampled at
the survivors' columns.
``maxk_forward`` / ``maxk_backward`` are the MaxK nonlinearity of the MaxK-GNN
review ("How MaxK-GNN works"): the dense [N, M] output that keeps each row's
exact top-k and zeroes the rest, and the gradient that flows back only to the
survivors' columns.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "rtopk_oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "librtopk_oracle.so")
# Host-sanitizer build (AddressSanitizer + UndefinedBehaviorSanitizer), used
# instead of the plain one when ORACLE_SANITIZE=1. Python is not built with
# ASan, so such a process needs the ASan runtime preloaded, e.g.
#   LD_PRELOAD=$(g++ -print-file-name=libasan.so) ASAN_OPTIONS=detect_leaks=0 \
#   ORACLE_SANITIZE=1 python -m pytest tests -m "not gpu"
_SAN_LIB_PATH = os.path.join(_HERE, "librtopk_oracle_san.so")
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer", "-g"]

_lib = None


def sanitized() -> bool:
    """Whether this process loads the sanitizer build (ORACLE_SANITIZE=1)."""
    return os.environ.get("ORACLE_SANITIZE", "") == "1"


def build(sanitize: bool | None = None) -> str:
    """Compile the oracle with g++ (IEEE single precision, no contraction).

    sanitize (default: ORACLE_SANITIZE=1) builds the separate copy with
    AddressSanitizer and UndefinedBehaviorSanitizer; the plain build is
    left as it is.
    """
    if sanitize is None:
        sanitize = sanitized()
    out = _SAN_LIB_PATH if sanitize else _LIB_PATH
    cmd = [
        "g++", "-std=c++17", "-O2", "-fopenmp", "-ffp-contract=off",
        "-fno-fast-math", "-fPIC", "-shared", *(_SAN_FLAGS if sanitize else []),
        "-o", out + ".tmp", _SRC,
    ]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = _SAN_LIB_PATH if sanitized() else _LIB_PATH
    if sanitized() or not os.path.exists(path):
        build()
    lib = ctypes.CDLL(path)
    f32p = ctypes.POINTER(ctypes.c_float)
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.oracle_exact.argtypes = [f32p, ctypes.c_int64, ctypes.c_int32,
                                 ctypes.c_int32, f32p, i32p]
    lib.oracle_exact.restype = ctypes.c_int
    lib.oracle_exact_by_sort.argtypes = [f32p, ctypes.c_int64, ctypes.c_int32,
                                         ctypes.c_int32, f32p, i32p]
    lib.oracle_exact_by_sort.restype = ctypes.c_int
    lib.oracle_capped.argtypes = [f32p, ctypes.c_int64, ctypes.c_int32,
                                  ctypes.c_int32, ctypes.c_int32,
                                  ctypes.c_float, ctypes.c_int32, f32p, i32p,
                                  i32p, f32p, f32p]
    lib.oracle_capped.restype = ctypes.c_int
    lib.oracle_bucketed.argtypes = [f32p, ctypes.c_int64, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, f32p, i32p]
    lib.oracle_bucketed.restype = ctypes.c_int
    lib.oracle_maxk_forward.argtypes = [f32p, ctypes.c_int64, ctypes.c_int32,
                                        ctypes.c_int32, f32p, f32p, i32p]
    lib.oracle_maxk_forward.restype = ctypes.c_int
    lib.oracle_maxk_backward.argtypes = [f32p, i32p, ctypes.c_int64,
                                         ctypes.c_int32, ctypes.c_int32, f32p]
    lib.oracle_maxk_backward.restype = ctypes.c_int
    i64p = ctypes.POINTER(ctypes.c_int64)
    lib.oracle_spgemm.argtypes = [i64p, i32p, f32p, ctypes.c_int64, ctypes.c_int64,
                                  f32p, i32p, ctypes.c_int32, ctypes.c_int32,
                                  f32p, f32p]
    lib.oracle_spgemm.restype = ctypes.c_int
    lib.oracle_sspmm.argtypes = [i64p, i32p, f32p, ctypes.c_int64, ctypes.c_int64,
                                 f32p, i32p, ctypes.c_int32, ctypes.c_int32,
                                 f32p, f32p]
    lib.oracle_sspmm.restype = ctypes.c_int
    lib.oracle_threads.argtypes = []
    lib.oracle_threads.restype = ctypes.c_int
    lib.oracle_set_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_threads.restype = None
    _lib = lib
    return lib


def _as_rows(x) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("x must be a 2-D [N, M] array")
    return x


def _fp(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _ip(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def exact(x, k: int):
    """Exact top-k of every row: (values [N,k] f32, indices [N,k] i32).

    The k-th largest value of each row comes from a partial selection
    (std::nth_element); survivors are the values above it, then the lowest
    columns holding it."""
    return _exact_with("oracle_exact", x, k)


def exact_by_sort(x, k: int):
    """The same result as ``exact`` through a full stable sort of each row
    (a second, independent path for the tests)."""
    return _exact_with("oracle_exact_by_sort", x, k)


def _exact_with(fn: str, x, k: int):
    x = _as_rows(x)
    n, m = x.shape
    vals = np.empty((n, k), dtype=np.float32)
    idx = np.empty((n, k), dtype=np.int32)
    rc = getattr(_load(), fn)(_fp(x), n, m, k, _fp(vals), _ip(idx))
    if rc != 0:
        raise ValueError(f"{fn}: invalid arguments (N={n}, M={m}, k={k})")
    return vals, idx


def capped(x, k: int, max_iter: int = -1, eps: float = 0.0,
           fill_from_row_min: bool = False, return_state: bool = False):
    """Capped threshold search with tie fill.

    Returns (values, indices) or, with ``return_state``, (values, indices,
    counts, lo, hi) where counts is the number of counts each row performed
    and [lo, hi] its final search bounds.
    """
    x = _as_rows(x)
    n, m = x.shape
    vals = np.empty((n, k), dtype=np.float32)
    idx = np.empty((n, k), dtype=np.int32)
    counts = np.empty((n,), dtype=np.int32)
    lo = np.empty((n,), dtype=np.float32)
    hi = np.empty((n,), dtype=np.float32)
    rc = _load().oracle_capped(_fp(x), n, m, k, int(max_iter),
                               ctypes.c_float(eps), int(bool(fill_from_row_min)),
                               _fp(vals), _ip(idx), _ip(counts), _fp(lo), _fp(hi))
    if rc != 0:
        raise ValueError(
            f"oracle_capped: invalid arguments (N={n}, M={m}, k={k}, eps={eps})")
    if return_state:
        return vals, idx, counts, lo, hi
    return vals, idx


def bucketed(x, k: int, buckets: int):
    """Bucketed top-k: (values [N,k] f32, indices [N,k] i32), bucket by bucket."""
    x = _as_rows(x)
    n, m = x.shape
    vals = np.empty((n, k), dtype=np.float32)
    idx = np.empty((n, k), dtype=np.int32)
    rc = _load().oracle_bucketed(_fp(x), n, m, k, int(buckets), _fp(vals), _ip(idx))
    if rc != 0:
        raise ValueError(f"oracle_bucketed: invalid arguments (N={n}, M={m}, k={k}, buckets={buckets})")
    return vals, idx


def maxk_forward(x, k: int):
    """MaxK nonlinearity: (y [N,M], sp_data [N,k], sp_index [N,k] i32)."""
    x = _as_rows(x)
    n, m = x.shape
    y = np.empty((n, m), dtype=np.float32)
    vals = np.empty((n, k), dtype=np.float32)
    idx = np.empty((n, k), dtype=np.int32)
    rc = _load().oracle_maxk_forward(_fp(x), n, m, k, _fp(y), _fp(vals), _ip(idx))
    if rc != 0:
        raise ValueError(f"oracle_maxk_forward: invalid arguments (N={n}, M={m}, k={k})")
    return y, vals, idx


def maxk_backward(grad_sp, sp_index, m: int):
    """Gradient of the MaxK survivors sent back to their columns: [N, m]."""
    g = np.ascontiguousarray(grad_sp, dtype=np.float32)
    idx = np.ascontiguousarray(sp_index, dtype=np.int32)
    if g.ndim != 2 or g.shape != idx.shape:
        raise ValueError("grad_sp and sp_index must be [N, k] arrays of one shape")
    n, k = g.shape
    out = np.empty((n, m), dtype=np.float32)
    rc = _load().oracle_maxk_backward(_fp(g), _ip(idx), n, m, k, _fp(out))
    if rc != 0:
        raise ValueError(f"oracle_maxk_backward: invalid arguments (N={n}, M={m}, k={k})")
    return out


def spgemm(row_ptr, col_idx, val, n_src: int, sp_data, sp_index, m: int,
           return_absum: bool = False):
    """Y [n_dst, m] = A X; with ``return_absum`` also sum |a x| per element."""
    rp = np.ascontiguousarray(row_ptr, dtype=np.int64)
    ci = np.ascontiguousarray(col_idx, dtype=np.int32)
    va = np.ascontiguousarray(val, dtype=np.float32)
    sd = np.ascontiguousarray(sp_data, dtype=np.float32)
    si = np.ascontiguousarray(sp_index, dtype=np.int32)
    n_dst = rp.shape[0] - 1
    k = sd.shape[1]
    if sd.shape != si.shape or sd.shape[0] != n_src or ci.shape != va.shape:
        raise ValueError("inconsistent shapes")
    y = np.empty((n_dst, m), dtype=np.float32)
    ab = np.empty((n_dst, m), dtype=np.float32) if return_absum else None
    rc = _load().oracle_spgemm(
        rp.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _ip(ci), _fp(va),
        n_dst, n_src, _fp(sd), _ip(si), m, k, _fp(y),
        _fp(ab) if ab is not None else None)
    if rc != 0:
        raise ValueError("oracle_spgemm: invalid arguments")
    return (y, ab) if return_absum else y


def sspmm(row_ptr, col_idx, val, dy, sp_index, return_absum: bool = False):
    """grad_sp [n_src, k] = (A^T dy) at the survivors' columns sp_index."""
    rp = np.ascontiguousarray(row_ptr, dtype=np.int64)
    ci = np.ascontiguousarray(col_idx, dtype=np.int32)
    va = np.ascontiguousarray(val, dtype=np.float32)
    g = np.ascontiguousarray(dy, dtype=np.float32)
    si = np.ascontiguousarray(sp_index, dtype=np.int32)
    n_dst = rp.shape[0] - 1
    n_src, k = si.shape
    if g.ndim != 2 or g.shape[0] != n_dst or ci.shape != va.shape:
        raise ValueError("inconsistent shapes")
    m = g.shape[1]
    out = np.empty((n_src, k), dtype=np.float32)
    ab = np.empty((n_src, k), dtype=np.float32) if return_absum else None
    rc = _load().oracle_sspmm(
        rp.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)), _ip(ci), _fp(va),
        n_dst, n_src, _fp(g), _ip(si), m, k, _fp(out),
        _fp(ab) if ab is not None else None)
    if rc != 0:
        raise ValueError("oracle_sspmm: invalid arguments")
    return (out, ab) if return_absum else out


def threads() -> int:
    """Threads the oracle's parallel loops use (OpenMP over rows)."""
    return int(_load().oracle_threads())


def set_threads(n: int) -> None:
    """Run the oracle's later calls on n threads (n >= 1)."""
    if n < 1:
        raise ValueError("set_threads: n must be at least 1")
    _load().oracle_set_threads(int(n))
