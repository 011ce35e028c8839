"""ctypes binding of librtopk.so (the C ABI declared in include/rtopk.h).

Argument marshalling only: every function here checks tensor shapes, dtypes
and devices, allocates outputs with torch when none are given, passes raw
device pointers and torch's current HIP stream, and maps status codes to
Python exceptions. All selection work runs in the library's HIP kernels; there
is no fallback path. If the library has not been built, every call raises.
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librtopk.so")

RTOPK_SUCCESS = 0
RTOPK_ERROR_INVALID_VALUE = 1
RTOPK_ERROR_NOT_SUPPORTED = 2
RTOPK_ERROR_LAUNCH = 3
RTOPK_MAX_ROW_LENGTH = 8192

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library, with argument types set. Raises if not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m row_wise_top_amd.build` "
            "(or __graft_entry__.build()); there is no fallback implementation")
    l = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    l.rtopk_select.argtypes = [vp, i64, i32, i32, i32, f32, vp, vp, vp]
    l.rtopk_select_u8.argtypes = [vp, i64, i32, i32, i32, f32, vp, vp, vp]
    l.rtopk_select_exact.argtypes = [vp, i64, i32, i32, vp, vp, vp]
    l.rtopk_select_exact_u8.argtypes = [vp, i64, i32, i32, vp, vp, vp]
    for f in (l.rtopk_select, l.rtopk_select_u8, l.rtopk_select_exact,
              l.rtopk_select_exact_u8):
        f.restype = ctypes.c_int
    l.rtopk_status_string.argtypes = [ctypes.c_int]
    l.rtopk_status_string.restype = ctypes.c_char_p
    _lib = l
    return l


def rtopk_status_string(status: int) -> str:
    return lib().rtopk_status_string(int(status)).decode()


def _check(status: int, what: str) -> None:
    if status == RTOPK_SUCCESS:
        return
    msg = f"{what}: {rtopk_status_string(status)}"
    if status == RTOPK_ERROR_INVALID_VALUE:
        raise ValueError(msg)
    if status == RTOPK_ERROR_NOT_SUPPORTED:
        raise NotImplementedError(msg)
    raise RuntimeError(msg)


def _prepare(x, k, out_val, out_idx, index_dtype):
    import torch
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda":
        raise ValueError("x must be a torch tensor on a GPU device")
    if x.dtype != torch.float32 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous 2-D float32 tensor [N, M]")
    n, m = x.shape
    if out_val is None:
        out_val = torch.empty((n, k), dtype=torch.float32, device=x.device)
    if out_idx is None:
        out_idx = torch.empty((n, k), dtype=index_dtype, device=x.device)
    for t, dt in ((out_val, torch.float32), (out_idx, index_dtype)):
        if (t.device != x.device or t.dtype != dt or not t.is_contiguous()
                or tuple(t.shape) != (n, k)):
            raise ValueError(f"outputs must be contiguous [{n}, {k}] {dt} on {x.device}")
    return n, m, out_val, out_idx


def _stream(x, stream):
    import torch
    if stream is None:
        return torch.cuda.current_stream(x.device).cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def rtopk_select(x, k: int, max_iter: int = -1, eps: float = 0.0,
                 out_val=None, out_idx=None, stream=None):
    """Capped threshold search with tie fill; int32 indices. Returns (values, indices)."""
    import torch
    n, m, out_val, out_idx = _prepare(x, k, out_val, out_idx, torch.int32)
    _check(lib().rtopk_select(x.data_ptr(), n, m, k, max_iter, eps,
                              out_val.data_ptr(), out_idx.data_ptr(),
                              _stream(x, stream)), "rtopk_select")
    return out_val, out_idx


def rtopk_select_u8(x, k: int, max_iter: int = -1, eps: float = 0.0,
                    out_val=None, out_idx=None, stream=None):
    """As rtopk_select with uint8 indices (M <= 256)."""
    import torch
    n, m, out_val, out_idx = _prepare(x, k, out_val, out_idx, torch.uint8)
    _check(lib().rtopk_select_u8(x.data_ptr(), n, m, k, max_iter, eps,
                                 out_val.data_ptr(), out_idx.data_ptr(),
                                 _stream(x, stream)), "rtopk_select_u8")
    return out_val, out_idx


def rtopk_select_exact(x, k: int, out_val=None, out_idx=None, stream=None):
    """Exact top-k (lowest index wins ties); int32 indices."""
    import torch
    n, m, out_val, out_idx = _prepare(x, k, out_val, out_idx, torch.int32)
    _check(lib().rtopk_select_exact(x.data_ptr(), n, m, k, out_val.data_ptr(),
                                    out_idx.data_ptr(), _stream(x, stream)),
           "rtopk_select_exact")
    return out_val, out_idx


def rtopk_select_exact_u8(x, k: int, out_val=None, out_idx=None, stream=None):
    """Exact top-k with uint8 indices (M <= 256)."""
    import torch
    n, m, out_val, out_idx = _prepare(x, k, out_val, out_idx, torch.uint8)
    _check(lib().rtopk_select_exact_u8(x.data_ptr(), n, m, k, out_val.data_ptr(),
                                       out_idx.data_ptr(), _stream(x, stream)),
           "rtopk_select_exact_u8")
    return out_val, out_idx
