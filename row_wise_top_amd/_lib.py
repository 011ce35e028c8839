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
    l.rtopk_select_bucketed.argtypes = [vp, i64, i32, i32, i32, vp, vp, vp]
    l.rtopk_select_bucketed_u8.argtypes = [vp, i64, i32, i32, i32, vp, vp, vp]
    l.rtopk_maxk_forward.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp]
    l.rtopk_maxk_forward_u8.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp]
    l.rtopk_maxk_backward.argtypes = [vp, vp, i64, i32, i32, vp, vp]
    l.rtopk_cbsr_spgemm.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, i32, i32, vp, vp]
    l.rtopk_cbsr_spgemm_u8.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, i32, i32, vp, vp]
    l.rtopk_cbsr_sspmm.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, i32, i32, vp, vp]
    l.rtopk_cbsr_sspmm_u8.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, i32, i32, vp, vp]
    l.rtopk_maxk_backward_u8.argtypes = [vp, vp, i64, i32, i32, vp, vp]
    for f in (l.rtopk_select, l.rtopk_select_u8, l.rtopk_select_exact,
              l.rtopk_select_exact_u8, l.rtopk_select_bucketed,
              l.rtopk_select_bucketed_u8, l.rtopk_maxk_forward,
              l.rtopk_maxk_forward_u8, l.rtopk_maxk_backward,
              l.rtopk_maxk_backward_u8, l.rtopk_cbsr_spgemm,
              l.rtopk_cbsr_spgemm_u8, l.rtopk_cbsr_sspmm, l.rtopk_cbsr_sspmm_u8):
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
    # Device indices as ints: cheaper than comparing torch.device objects on
    # every call of a small batch.
    dev = x.get_device()
    for t, dt in ((out_val, torch.float32), (out_idx, index_dtype)):
        if (not t.is_cuda or t.get_device() != dev or t.dtype != dt
                or not t.is_contiguous() or t.shape != (n, k)):
            raise ValueError(f"outputs must be contiguous [{n}, {k}] {dt} on {x.device}")
    return n, m, out_val, out_idx


def _stream(x, stream):
    """The HIP stream handle to enqueue on: torch's current stream of x's
    device unless one is given (a torch stream or a raw handle)."""
    import torch
    if stream is None:
        # The raw handle straight from torch's stream registry when this
        # torch has the accessor (no Stream object built per call).
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:
            return raw(x.get_device())
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


def rtopk_select_bucketed(x, k: int, buckets: int, out_val=None, out_idx=None,
                          index_dtype=None, stream=None):
    """Bucketed top-k: the exact top-(k/buckets) of each of `buckets`
    contiguous buckets of every row, columns relative to the row, bucket by
    bucket. index_dtype: torch.int32 (default) or torch.uint8 (M <= 256)."""
    import torch
    idx_dtype = torch.int32 if index_dtype is None else index_dtype
    if idx_dtype not in (torch.int32, torch.uint8):
        raise ValueError("index_dtype must be torch.int32 or torch.uint8")
    n, m, out_val, out_idx = _prepare(x, k, out_val, out_idx, idx_dtype)
    u8 = idx_dtype == torch.uint8
    fn = lib().rtopk_select_bucketed_u8 if u8 else lib().rtopk_select_bucketed
    _check(fn(x.data_ptr(), n, m, k, int(buckets), out_val.data_ptr(),
              out_idx.data_ptr(), _stream(x, stream)),
           "rtopk_select_bucketed_u8" if u8 else "rtopk_select_bucketed")
    return out_val, out_idx


def rtopk_maxk_forward(x, k: int, y=None, sp_data=None, sp_index=None,
                       index_dtype=None, stream=None):
    """MaxK nonlinearity: (y [N, M] with each row's exact top-k kept and the
    rest zero, sp_data [N, k], sp_index [N, k]). index_dtype: torch.int32
    (default) or torch.uint8 (M <= 256)."""
    import torch
    idx_dtype = torch.int32 if index_dtype is None else index_dtype
    if idx_dtype not in (torch.int32, torch.uint8):
        raise ValueError("index_dtype must be torch.int32 or torch.uint8")
    n, m, sp_data, sp_index = _prepare(x, k, sp_data, sp_index, idx_dtype)
    if y is None:
        y = torch.empty((n, m), dtype=torch.float32, device=x.device)
    if (y.device != x.device or y.dtype != torch.float32 or not y.is_contiguous()
            or tuple(y.shape) != (n, m)):
        raise ValueError(f"y must be a contiguous [{n}, {m}] float32 tensor on {x.device}")
    u8 = idx_dtype == torch.uint8
    fn = lib().rtopk_maxk_forward_u8 if u8 else lib().rtopk_maxk_forward
    _check(fn(x.data_ptr(), n, m, k, y.data_ptr(), sp_data.data_ptr(),
              sp_index.data_ptr(), _stream(x, stream)),
           "rtopk_maxk_forward_u8" if u8 else "rtopk_maxk_forward")
    return y, sp_data, sp_index


def rtopk_maxk_backward(grad_sp, sp_index, m: int, grad_x=None, stream=None):
    """Dense [N, m] gradient of the MaxK survivors: grad_x[r, sp_index[r, i]] =
    grad_sp[r, i], zero elsewhere. sp_index is int32 or uint8 (m <= 256)."""
    import torch
    for t in (grad_sp, sp_index):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError("grad_sp and sp_index must be torch tensors on a GPU device")
    if (grad_sp.dtype != torch.float32 or grad_sp.dim() != 2
            or not grad_sp.is_contiguous()):
        raise ValueError("grad_sp must be a contiguous 2-D float32 tensor [N, k]")
    if (sp_index.dtype not in (torch.int32, torch.uint8) or not sp_index.is_contiguous()
            or tuple(sp_index.shape) != tuple(grad_sp.shape)
            or sp_index.device != grad_sp.device):
        raise ValueError("sp_index must be a contiguous int32 or uint8 tensor shaped like grad_sp")
    n, k = grad_sp.shape
    if grad_x is None:
        grad_x = torch.empty((n, m), dtype=torch.float32, device=grad_sp.device)
    if (grad_x.device != grad_sp.device or grad_x.dtype != torch.float32
            or not grad_x.is_contiguous() or tuple(grad_x.shape) != (n, m)):
        raise ValueError(f"grad_x must be a contiguous [{n}, {m}] float32 tensor on {grad_sp.device}")
    u8 = sp_index.dtype == torch.uint8
    fn = lib().rtopk_maxk_backward_u8 if u8 else lib().rtopk_maxk_backward
    _check(fn(grad_sp.data_ptr(), sp_index.data_ptr(), n, m, k, grad_x.data_ptr(),
              _stream(grad_sp, stream)),
           "rtopk_maxk_backward_u8" if u8 else "rtopk_maxk_backward")
    return grad_x


def rtopk_cbsr_spgemm(row_ptr, col_idx, val, sp_data, sp_index, m: int, y=None,
                      stream=None):
    """MaxK-GNN aggregation y = A X: A in CSR (row_ptr int64 [n_dst + 1],
    col_idx int32 [nnz], val float32 [nnz]), X as compressed rows (sp_data
    float32 [n_src, k], sp_index int32 or uint8 [n_src, k], m columns).
    Returns y, float32 [n_dst, m]."""
    import torch
    for t, dt, name in ((row_ptr, (torch.int64,), "row_ptr"), (col_idx, (torch.int32,), "col_idx"),
                        (val, (torch.float32,), "val"), (sp_data, (torch.float32,), "sp_data"),
                        (sp_index, (torch.int32, torch.uint8), "sp_index")):
        if (not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype not in dt
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous GPU tensor of dtype {dt}")
    if row_ptr.dim() != 1 or col_idx.dim() != 1 or val.shape != col_idx.shape:
        raise ValueError("row_ptr, col_idx and val must be 1-D, col_idx and val of one length")
    if sp_data.dim() != 2 or sp_index.shape != sp_data.shape:
        raise ValueError("sp_data and sp_index must be [n_src, k] tensors of one shape")
    n_dst = row_ptr.shape[0] - 1
    n_src, k = sp_data.shape
    nnz = col_idx.shape[0]
    if y is None:
        y = torch.empty((n_dst, m), dtype=torch.float32, device=sp_data.device)
    if (y.device != sp_data.device or y.dtype != torch.float32 or not y.is_contiguous()
            or tuple(y.shape) != (n_dst, m)):
        raise ValueError(f"y must be a contiguous [{n_dst}, {m}] float32 tensor")
    u8 = sp_index.dtype == torch.uint8
    fn = lib().rtopk_cbsr_spgemm_u8 if u8 else lib().rtopk_cbsr_spgemm
    _check(fn(row_ptr.data_ptr(), col_idx.data_ptr(), val.data_ptr(), n_dst, n_src, nnz,
              sp_data.data_ptr(), sp_index.data_ptr(), m, k, y.data_ptr(),
              _stream(sp_data, stream)),
           "rtopk_cbsr_spgemm_u8" if u8 else "rtopk_cbsr_spgemm")
    return y


def rtopk_cbsr_sspmm(row_ptr, col_idx, val, dy, sp_index, grad_sp=None, stream=None):
    """Backward of rtopk_cbsr_spgemm to the compressed features: grad_sp
    [n_src, k] = (A^T dy) at the survivors' columns sp_index (int32 or uint8,
    [n_src, k]); dy is float32 [n_dst, M]."""
    import torch
    for t, dt, name in ((row_ptr, (torch.int64,), "row_ptr"), (col_idx, (torch.int32,), "col_idx"),
                        (val, (torch.float32,), "val"), (dy, (torch.float32,), "dy"),
                        (sp_index, (torch.int32, torch.uint8), "sp_index")):
        if (not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype not in dt
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous GPU tensor of dtype {dt}")
    if row_ptr.dim() != 1 or col_idx.dim() != 1 or val.shape != col_idx.shape:
        raise ValueError("row_ptr, col_idx and val must be 1-D, col_idx and val of one length")
    n_dst = row_ptr.shape[0] - 1
    if dy.dim() != 2 or dy.shape[0] != n_dst or sp_index.dim() != 2:
        raise ValueError("dy must be [n_dst, M] and sp_index [n_src, k]")
    m = dy.shape[1]
    n_src, k = sp_index.shape
    if grad_sp is None:
        grad_sp = torch.empty((n_src, k), dtype=torch.float32, device=dy.device)
    if (grad_sp.device != dy.device or grad_sp.dtype != torch.float32
            or not grad_sp.is_contiguous() or tuple(grad_sp.shape) != (n_src, k)):
        raise ValueError(f"grad_sp must be a contiguous [{n_src}, {k}] float32 tensor")
    u8 = sp_index.dtype == torch.uint8
    fn = lib().rtopk_cbsr_sspmm_u8 if u8 else lib().rtopk_cbsr_sspmm
    _check(fn(row_ptr.data_ptr(), col_idx.data_ptr(), val.data_ptr(), n_dst, n_src,
              col_idx.shape[0], dy.data_ptr(), sp_index.data_ptr(), m, k,
              grad_sp.data_ptr(), _stream(dy, stream)),
           "rtopk_cbsr_sspmm_u8" if u8 else "rtopk_cbsr_sspmm")
    return grad_sp
