"""Row-wise top-k selection on MI355X (gfx950).

The selection runs in hand-written HIP kernels behind the C ABI of
include/rtopk.h (librtopk.so); this package is a thin binding over it.

    values, indices = row_wise_top_amd.select(x, k)            # exact
    values, indices = row_wise_top_amd.select(x, k, max_iter=4) # early stop
"""

from __future__ import annotations

from ._lib import (RTOPK_MAX_ROW_LENGTH, lib, rtopk_cbsr_spgemm, rtopk_cbsr_sspmm,
                   rtopk_maxk_backward,
                   rtopk_maxk_forward, rtopk_select, rtopk_select_bucketed,
                   rtopk_select_exact, rtopk_select_exact_u8, rtopk_select_u8,
                   rtopk_status_string)

__all__ = ["select", "lib", "rtopk_select", "rtopk_select_exact",
           "rtopk_select_u8", "rtopk_select_exact_u8", "rtopk_select_bucketed",
           "rtopk_maxk_forward",
           "rtopk_maxk_backward", "rtopk_cbsr_spgemm", "rtopk_cbsr_sspmm",
           "rtopk_status_string", "RTOPK_MAX_ROW_LENGTH"]


def select(x, k: int, max_iter: int = -1, eps: float = 0.0,
           exact: bool = False, index_dtype=None):
    """Top-k of every row of a [N, M] float32 GPU tensor.

    exact=True: the exact top-k (ties at the k-th value to the lowest
    indices). Otherwise the capped threshold search with tie fill, which is
    also exact when max_iter < 0 and eps == 0. Survivors come back in
    ascending column order. index_dtype: torch.int32 (default) or torch.uint8
    (rows of at most 256).
    """
    import torch
    u8 = index_dtype is not None and index_dtype == torch.uint8
    if exact:
        return rtopk_select_exact_u8(x, k) if u8 else rtopk_select_exact(x, k)
    if u8:
        return rtopk_select_u8(x, k, max_iter, eps)
    return rtopk_select(x, k, max_iter, eps)
