// C ABI of the row-wise top-k library: argument validation and dispatch.
// The operation and the argument contract are documented in include/rtopk.h.

#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "rtopk.h"
#include "rtopk_internal.h"

namespace {

rtopk_status_t validate(const float* x, int64_t n, int32_t m, int32_t k,
                        float eps, const float* out_val, const void* out_idx,
                        bool u8_index) {
  if (n < 0 || m < 1 || k < 1 || k > m) return RTOPK_ERROR_INVALID_VALUE;
  if (!(eps >= 0.0f)) return RTOPK_ERROR_INVALID_VALUE;  // rejects NaN too
  if (m > rtopk::kMaxRowLength) return RTOPK_ERROR_NOT_SUPPORTED;
  if (u8_index && m > 256) return RTOPK_ERROR_NOT_SUPPORTED;
  if (n > 0 && (x == nullptr || out_val == nullptr || out_idx == nullptr))
    return RTOPK_ERROR_INVALID_VALUE;
  return RTOPK_SUCCESS;
}

rtopk_status_t run(const float* x, int64_t n, int32_t m, int32_t k,
                   int32_t max_iter, float eps, float* out_val, void* out_idx,
                   bool u8_index, rtopk::Mode mode, hipStream_t stream) {
  const rtopk_status_t st =
      validate(x, n, m, k, eps, out_val, out_idx, u8_index);
  if (st != RTOPK_SUCCESS) return st;
  if (n == 0) return RTOPK_SUCCESS;
  rtopk::SelectArgs a{x, n, m, k, max_iter, eps, out_val, out_idx, 0.0f, 0.0f, nullptr, 1};
  // Short rows keeping few survivors, exact: one lane (or two) per row, 64
  // (or 32) rows per wave (the bucket kernels with one bucket per row),
  // instead of one row per wave with most lanes idle.
  const bool exact = mode == rtopk::Mode::kExact ||
                     (mode == rtopk::Mode::kCapped && max_iter < 0 && eps == 0.0f);
  const hipError_t err = exact && rtopk::bucket_lanes_supported(x, m, k)
                             ? rtopk::launch_bucket_lanes(a, u8_index, stream)
                             : rtopk::launch_select(a, mode, u8_index, stream);
  return err == hipSuccess ? RTOPK_SUCCESS : RTOPK_ERROR_LAUNCH;
}

rtopk_status_t run_scatter(const float* src, const void* idx, int64_t n,
                           int32_t m, int32_t k, float* out, bool u8_index,
                           hipStream_t stream) {
  if (n < 0 || m < 1 || k < 1 || k > m) return RTOPK_ERROR_INVALID_VALUE;
  if (m > rtopk::kMaxRowLength) return RTOPK_ERROR_NOT_SUPPORTED;
  if (u8_index && m > 256) return RTOPK_ERROR_NOT_SUPPORTED;
  if (n > 0 && (src == nullptr || idx == nullptr || out == nullptr))
    return RTOPK_ERROR_INVALID_VALUE;
  if (n == 0) return RTOPK_SUCCESS;
  const rtopk::ScatterArgs a{src, idx, n, m, k, out};
  const hipError_t err = rtopk::launch_scatter(a, u8_index, stream);
  return err == hipSuccess ? RTOPK_SUCCESS : RTOPK_ERROR_LAUNCH;
}

// MaxK forward: the exact selection with the dense output. Rows the fused
// kernel takes in one launch; longer rows run the selection into (sp_data,
// sp_index) and then scatter those into y, on the same stream.
rtopk_status_t run_maxk_forward(const float* x, int64_t n, int32_t m, int32_t k,
                                float* y, float* sp_data, void* sp_index,
                                bool u8_index, hipStream_t stream) {
  const rtopk_status_t st =
      validate(x, n, m, k, 0.0f, sp_data, sp_index, u8_index);
  if (st != RTOPK_SUCCESS) return st;
  if (n > 0 && y == nullptr) return RTOPK_ERROR_INVALID_VALUE;
  if (n == 0) return RTOPK_SUCCESS;
  const int q = (m + rtopk::kWave - 1) / rtopk::kWave;
  rtopk::SelectArgs a{x, n, m, k, -1, 0.0f, sp_data, sp_index, 0.0f, 0.0f, y, 1};
  hipError_t err;
  if (rtopk::maxk_fused(q)) {
    err = rtopk::launch_select(a, rtopk::Mode::kMaxk, u8_index, stream);
  } else {
    a.dense = nullptr;
    err = rtopk::launch_select(a, rtopk::Mode::kExact, u8_index, stream);
    if (err == hipSuccess) {
      const rtopk::ScatterArgs s{sp_data, sp_index, n, m, k, y};
      err = rtopk::launch_scatter(s, u8_index, stream);
    }
  }
  return err == hipSuccess ? RTOPK_SUCCESS : RTOPK_ERROR_LAUNCH;
}

// Bucketed top-k over the [n * buckets, m / buckets] view of x (each bucket
// a row, k / buckets survivors), emitted columns offset by the bucket's
// position; the [n, k] outputs are the [n * buckets, k / buckets] outputs of
// that view. Short buckets take one lane each (rtopk_bucket.hip), longer
// ones the exact wave-per-row kernel.
rtopk_status_t run_bucketed(const float* x, int64_t n, int32_t m, int32_t k,
                            int32_t buckets, float* out_val, void* out_idx,
                            bool u8_index, hipStream_t stream) {
  const rtopk_status_t st = validate(x, n, m, k, 0.0f, out_val, out_idx, u8_index);
  if (st != RTOPK_SUCCESS) return st;
  if (buckets < 1 || m % buckets != 0 || k % buckets != 0)
    return RTOPK_ERROR_INVALID_VALUE;
  const int32_t width = m / buckets;
  if (!rtopk::bucket_supported((width + rtopk::kWave - 1) / rtopk::kWave))
    return RTOPK_ERROR_NOT_SUPPORTED;
  if (n > INT64_MAX / buckets) return RTOPK_ERROR_NOT_SUPPORTED;
  if (n == 0) return RTOPK_SUCCESS;
  rtopk::SelectArgs a{x,       n * buckets, width, k / buckets, -1, 0.0f,
                      out_val, out_idx,     0.0f,  0.0f,        nullptr, buckets};
  const hipError_t err =
      rtopk::bucket_lanes_supported(x, width, k / buckets)
          ? rtopk::launch_bucket_lanes(a, u8_index, stream)
          : rtopk::launch_select(a, rtopk::Mode::kBucket, u8_index, stream);
  return err == hipSuccess ? RTOPK_SUCCESS : RTOPK_ERROR_LAUNCH;
}

rtopk_status_t run_spgemm(const int64_t* row_ptr, const int32_t* col,
                          const float* val, int64_t n_dst, int64_t n_src,
                          int64_t nnz, const float* sp_data, const void* sp_index,
                          int32_t m, int32_t k, float* y, bool u8_index,
                          hipStream_t stream) {
  if (n_dst < 0 || n_src < 0 || nnz < 0 || m < 1 || k < 1 || k > m)
    return RTOPK_ERROR_INVALID_VALUE;
  if (nnz > 0 && n_src < 1) return RTOPK_ERROR_INVALID_VALUE;
  if (m > rtopk::kMaxRowLength) return RTOPK_ERROR_NOT_SUPPORTED;
  if (u8_index && m > 256) return RTOPK_ERROR_NOT_SUPPORTED;
  if (n_dst > 0 && (row_ptr == nullptr || y == nullptr)) return RTOPK_ERROR_INVALID_VALUE;
  if (nnz > 0 && (col == nullptr || val == nullptr || sp_data == nullptr ||
                  sp_index == nullptr))
    return RTOPK_ERROR_INVALID_VALUE;
  if (n_dst == 0) return RTOPK_SUCCESS;
  rtopk::SpgemmArgs a{row_ptr, col, val, n_dst, n_src, nnz, sp_data, sp_index,
                      m, k, y, 0, 0, 0, 0, 0};
  const hipError_t err = rtopk::launch_spgemm(a, u8_index, stream);
  return err == hipSuccess ? RTOPK_SUCCESS : RTOPK_ERROR_LAUNCH;
}

rtopk_status_t run_sspmm(const int64_t* row_ptr, const int32_t* col,
                         const float* val, int64_t n_dst, int64_t n_src,
                         int64_t nnz, const float* dy, const void* sp_index,
                         int32_t m, int32_t k, float* grad_sp, bool u8_index,
                         hipStream_t stream) {
  if (n_dst < 0 || n_src < 0 || nnz < 0 || m < 1 || k < 1 || k > m)
    return RTOPK_ERROR_INVALID_VALUE;
  if (nnz > 0 && n_src < 1) return RTOPK_ERROR_INVALID_VALUE;
  if (m > rtopk::kMaxRowLength) return RTOPK_ERROR_NOT_SUPPORTED;
  if (u8_index && m > 256) return RTOPK_ERROR_NOT_SUPPORTED;
  if (n_src > 0 && grad_sp == nullptr) return RTOPK_ERROR_INVALID_VALUE;
  if (nnz > 0 && (row_ptr == nullptr || col == nullptr || val == nullptr ||
                  dy == nullptr || sp_index == nullptr))
    return RTOPK_ERROR_INVALID_VALUE;
  if (n_src == 0) return RTOPK_SUCCESS;
  rtopk::SpgemmArgs a{row_ptr, col, val, n_dst, n_src, nnz, dy, sp_index,
                      m, k, grad_sp, 0, 0, 0, 0, 0};
  const hipError_t err = rtopk::launch_sspmm(a, u8_index, stream);
  return err == hipSuccess ? RTOPK_SUCCESS : RTOPK_ERROR_LAUNCH;
}

}  // namespace

extern "C" {

rtopk_status_t rtopk_select(const float* x, int64_t N, int32_t M, int32_t k,
                            int32_t max_iter, float eps, float* out_val,
                            int32_t* out_idx, hipStream_t stream) {
  return run(x, N, M, k, max_iter, eps, out_val, out_idx, false,
             rtopk::Mode::kCapped, stream);
}

rtopk_status_t rtopk_select_exact(const float* x, int64_t N, int32_t M,
                                  int32_t k, float* out_val, int32_t* out_idx,
                                  hipStream_t stream) {
  return run(x, N, M, k, -1, 0.0f, out_val, out_idx, false,
             rtopk::Mode::kExact, stream);
}

rtopk_status_t rtopk_select_u8(const float* x, int64_t N, int32_t M, int32_t k,
                               int32_t max_iter, float eps, float* out_val,
                               uint8_t* out_idx, hipStream_t stream) {
  return run(x, N, M, k, max_iter, eps, out_val, out_idx, true,
             rtopk::Mode::kCapped, stream);
}

rtopk_status_t rtopk_select_exact_u8(const float* x, int64_t N, int32_t M,
                                     int32_t k, float* out_val,
                                     uint8_t* out_idx, hipStream_t stream) {
  return run(x, N, M, k, -1, 0.0f, out_val, out_idx, true,
             rtopk::Mode::kExact, stream);
}

rtopk_status_t rtopk_select_bucketed(const float* x, int64_t N, int32_t M,
                                     int32_t k, int32_t buckets, float* out_val,
                                     int32_t* out_idx, hipStream_t stream) {
  return run_bucketed(x, N, M, k, buckets, out_val, out_idx, false, stream);
}

rtopk_status_t rtopk_select_bucketed_u8(const float* x, int64_t N, int32_t M,
                                        int32_t k, int32_t buckets,
                                        float* out_val, uint8_t* out_idx,
                                        hipStream_t stream) {
  return run_bucketed(x, N, M, k, buckets, out_val, out_idx, true, stream);
}

rtopk_status_t rtopk_maxk_forward(const float* x, int64_t N, int32_t M,
                                  int32_t k, float* y, float* sp_data,
                                  int32_t* sp_index, hipStream_t stream) {
  return run_maxk_forward(x, N, M, k, y, sp_data, sp_index, false, stream);
}

rtopk_status_t rtopk_maxk_forward_u8(const float* x, int64_t N, int32_t M,
                                     int32_t k, float* y, float* sp_data,
                                     uint8_t* sp_index, hipStream_t stream) {
  return run_maxk_forward(x, N, M, k, y, sp_data, sp_index, true, stream);
}

rtopk_status_t rtopk_cbsr_spgemm(const int64_t* row_ptr, const int32_t* col_idx,
                                 const float* val, int64_t n_dst, int64_t n_src,
                                 int64_t nnz, const float* sp_data,
                                 const int32_t* sp_index, int32_t M, int32_t k,
                                 float* y, hipStream_t stream) {
  return run_spgemm(row_ptr, col_idx, val, n_dst, n_src, nnz, sp_data, sp_index,
                    M, k, y, false, stream);
}

rtopk_status_t rtopk_cbsr_spgemm_u8(const int64_t* row_ptr, const int32_t* col_idx,
                                    const float* val, int64_t n_dst, int64_t n_src,
                                    int64_t nnz, const float* sp_data,
                                    const uint8_t* sp_index, int32_t M, int32_t k,
                                    float* y, hipStream_t stream) {
  return run_spgemm(row_ptr, col_idx, val, n_dst, n_src, nnz, sp_data, sp_index,
                    M, k, y, true, stream);
}

rtopk_status_t rtopk_cbsr_sspmm(const int64_t* row_ptr, const int32_t* col_idx,
                                const float* val, int64_t n_dst, int64_t n_src,
                                int64_t nnz, const float* dy,
                                const int32_t* sp_index, int32_t M, int32_t k,
                                float* grad_sp, hipStream_t stream) {
  return run_sspmm(row_ptr, col_idx, val, n_dst, n_src, nnz, dy, sp_index, M, k,
                   grad_sp, false, stream);
}

rtopk_status_t rtopk_cbsr_sspmm_u8(const int64_t* row_ptr, const int32_t* col_idx,
                                   const float* val, int64_t n_dst, int64_t n_src,
                                   int64_t nnz, const float* dy,
                                   const uint8_t* sp_index, int32_t M, int32_t k,
                                   float* grad_sp, hipStream_t stream) {
  return run_sspmm(row_ptr, col_idx, val, n_dst, n_src, nnz, dy, sp_index, M, k,
                   grad_sp, true, stream);
}

rtopk_status_t rtopk_maxk_backward(const float* grad_sp,
                                   const int32_t* sp_index, int64_t N,
                                   int32_t M, int32_t k, float* grad_x,
                                   hipStream_t stream) {
  return run_scatter(grad_sp, sp_index, N, M, k, grad_x, false, stream);
}

rtopk_status_t rtopk_maxk_backward_u8(const float* grad_sp,
                                      const uint8_t* sp_index, int64_t N,
                                      int32_t M, int32_t k, float* grad_x,
                                      hipStream_t stream) {
  return run_scatter(grad_sp, sp_index, N, M, k, grad_x, true, stream);
}

const char* rtopk_status_string(rtopk_status_t status) {
  switch (status) {
    case RTOPK_SUCCESS:
      return "success";
    case RTOPK_ERROR_INVALID_VALUE:
      return "invalid value: null pointer, N < 0, M < 1, k < 1, k > M, eps < 0 / NaN, "
             "or buckets that do not divide M and k";
    case RTOPK_ERROR_NOT_SUPPORTED:
      return "not supported: M > 8192, one-byte indices with M > 256, or buckets "
             "longer than 1024";
    case RTOPK_ERROR_LAUNCH:
      return "kernel launch failed";
  }
  return "unknown status";
}

}  // extern "C"
