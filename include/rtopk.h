/*
 * rtopk.h -- C ABI of the row-wise top-k library for MI355X (gfx950).
 *
 * Operation. For every row of a row-major [N, M] single-precision matrix,
 * select k of its M elements and write them, unsorted by value, as two dense
 * row-major [N, k] arrays: the selected values and their column indices. This
 * is the row-wise top-k of the RTop-K summary page ("RTop-K: Ultra-Fast
 * Row-Wise Top-K Selection for Neural Network Acceleration on GPUs", sections
 * "Problem" and "Approach"), whose output is the two-array compressed
 * balanced layout (data + index, exactly k per row) of the MaxK-GNN review
 * ("MaxK-GNN: Extremely Fast GPU Kernel Design ...", section "How MaxK-GNN
 * works") and the MaxK-GNN abstract (CBSR format).
 *
 * Output order. Within a row the k survivors are listed in ascending column
 * index. Both the exact and the capped entry points write exactly k entries
 * per row; out_idx[r*k + i] is a distinct column in [0, M) and
 * out_val[r*k + i] is bitwise x[r*M + out_idx[r*k + i]].
 *
 * Arguments common to every entry point.
 *   x        device pointer to N*M floats, row r at x + r*M (no padding).
 *            Elements must be finite; NaN or infinity gives an unspecified
 *            (but in-bounds) selection. -0.0 and +0.0 compare equal.
 *   N        number of rows, N >= 0. N == 0 returns RTOPK_SUCCESS and
 *            launches nothing. 64-bit: inputs beyond 4 GiB are supported.
 *   M        row length, 1 <= M <= RTOPK_MAX_ROW_LENGTH (8192; the summary
 *            page, "Limitations", reports the method unsupported beyond it).
 *   k        survivors per row, 1 <= k <= M.
 *   out_val  device pointer to N*k floats, written.
 *   out_idx  device pointer to N*k indices (int32, or uint8 for the _u8
 *            forms), written.
 *   stream   HIP stream to enqueue on; NULL means the null stream.
 * Outputs must not overlap x or each other. All pointers are owned by the
 * caller; the library allocates, frees and synchronises nothing, and keeps no
 * state between calls apart from cached device properties and, per calling
 * thread, the host-side search constants of the last (M, k) (re-entrant).
 *
 * Asynchrony. Each call validates its arguments on the host, enqueues its
 * kernel on `stream` (two kernels, in order, for the calls that say so:
 * rtopk_maxk_forward on rows longer than 1,024, rtopk_cbsr_spgemm and
 * rtopk_cbsr_sspmm) and returns. Faults in a kernel surface at the caller's
 * next synchronisation, as for any HIP launch.
 *
 * Errors. RTOPK_ERROR_INVALID_VALUE: a NULL pointer (when N > 0), N < 0,
 * M < 1, k < 1, k > M, eps < 0 or NaN (and the bucket conditions below).
 * RTOPK_ERROR_NOT_SUPPORTED: M > RTOPK_MAX_ROW_LENGTH, or a _u8 form with
 * M > 256 (and buckets longer than 1024). With either of these nothing is
 * enqueued and the outputs are untouched: every argument and launch
 * configuration is checked before the first launch. RTOPK_ERROR_LAUNCH: the
 * HIP runtime reported an error while enqueuing (hipGetLastError after a
 * launch). A one-kernel call then has enqueued nothing. A two-kernel call
 * checks each launch before the next, so nothing follows a failed launch;
 * but when the second launch fails, the first kernel (the selection, or the
 * zeroing kernel of the aggregation calls) is already enqueued and the
 * outputs are unspecified.
 */
#ifndef RTOPK_H_
#define RTOPK_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RTOPK_MAX_ROW_LENGTH 8192

typedef enum rtopk_status_t {
  RTOPK_SUCCESS = 0,
  RTOPK_ERROR_INVALID_VALUE = 1,
  RTOPK_ERROR_NOT_SUPPORTED = 2,
  RTOPK_ERROR_LAUNCH = 3
} rtopk_status_t;

/*
 * Capped threshold search with tie fill (RTop-K summary page, "Approach";
 * early stopping in "Key results"; precision epsilon in "Surprising
 * findings"). Per row, in IEEE single precision with round-to-nearest-even:
 *   lo = min(row), hi = max(row), steps = 0
 *   while (max_iter < 0 || steps < max_iter):
 *     if (hi - lo <= eps) stop
 *     mid = 0.5f*lo + 0.5f*hi;  if !(lo < mid < hi) stop
 *     c = #{x >= mid}; steps += 1
 *     c == k: lo = hi = mid, stop;  c > k: lo = mid;  c < k: hi = mid
 *   survivors = first k (by index) of A = {x >= hi}, then of B = {lo <= x < hi}
 * max_iter < 0 means no cap; max_iter == 0 performs no count. eps is an
 * absolute width (eps >= 0). With max_iter < 0 and eps == 0 the result is the
 * exact top-k with ties at the k-th value broken by lowest index.
 */
rtopk_status_t rtopk_select(const float* x, int64_t N, int32_t M, int32_t k,
                            int32_t max_iter, float eps, float* out_val,
                            int32_t* out_idx, hipStream_t stream);

/*
 * Exact top-k (RTop-K summary page, "Problem": the k largest of each row),
 * without sorting: the threshold search runs until it isolates the k-th
 * largest value exactly, with a bounded number of counts per row. Ties at the
 * k-th value go to the lowest indices, so the result equals the first k
 * positions of a stable descending sort, re-listed by ascending index.
 */
rtopk_status_t rtopk_select_exact(const float* x, int64_t N, int32_t M,
                                  int32_t k, float* out_val, int32_t* out_idx,
                                  hipStream_t stream);

/* As rtopk_select with one-byte column indices (the compressed balanced
 * layout's index array for rows of at most 256 features). Requires M <= 256. */
rtopk_status_t rtopk_select_u8(const float* x, int64_t N, int32_t M, int32_t k,
                               int32_t max_iter, float eps, float* out_val,
                               uint8_t* out_idx, hipStream_t stream);

/* As rtopk_select_exact with one-byte column indices. Requires M <= 256. */
rtopk_status_t rtopk_select_exact_u8(const float* x, int64_t N, int32_t M,
                                     int32_t k, float* out_val,
                                     uint8_t* out_idx, hipStream_t stream);

/*
 * Bucketed approximate top-k (page "Approximate Top-k for Increased
 * Parallelism": independent small top-k selections in place of one). Each
 * row is cut into `buckets` contiguous buckets of M / buckets columns, each
 * bucket keeps its exact top (k / buckets) (ties to the lowest columns), and
 * the k survivors are written bucket by bucket, i.e. in ascending column
 * order, with columns relative to the whole row.
 *   buckets  1 <= buckets, M % buckets == 0 and k % buckets == 0
 *            (else RTOPK_ERROR_INVALID_VALUE); M / buckets <= 1024 (else
 *            RTOPK_ERROR_NOT_SUPPORTED).
 * Everything else is as for rtopk_select_exact; buckets == 1 is the exact
 * top-k.
 */
rtopk_status_t rtopk_select_bucketed(const float* x, int64_t N, int32_t M,
                                     int32_t k, int32_t buckets, float* out_val,
                                     int32_t* out_idx, hipStream_t stream);

/* As rtopk_select_bucketed with one-byte column indices. Requires M <= 256. */
rtopk_status_t rtopk_select_bucketed_u8(const float* x, int64_t N, int32_t M,
                                        int32_t k, int32_t buckets,
                                        float* out_val, uint8_t* out_idx,
                                        hipStream_t stream);

/*
 * MaxK nonlinearity, forward (MaxK-GNN review, "How MaxK-GNN works": each row
 * keeps exactly its k largest features and every other feature becomes zero;
 * the survivors are also kept as the compressed pair sp_data / sp_index that
 * the aggregation and the backward pass consume). Per row, the survivors are
 * those of rtopk_select_exact (ties at the k-th value to the lowest columns)
 * and
 *   y[r*M + j] = x[r*M + j]   (bit copy) if column j survives, else +0.0,
 *   sp_data / sp_index        as out_val / out_idx of rtopk_select_exact.
 *   y         device pointer to N*M floats, written (every element).
 *   sp_data   device pointer to N*k floats, written.
 *   sp_index  device pointer to N*k int32 (uint8 for the _u8 form), written.
 * x, N, M, k, stream and the errors are as above. Rows of at most 1024
 * elements take one kernel; longer rows take two, enqueued on `stream` in
 * order. y must not overlap x or the other outputs.
 */
rtopk_status_t rtopk_maxk_forward(const float* x, int64_t N, int32_t M,
                                  int32_t k, float* y, float* sp_data,
                                  int32_t* sp_index, hipStream_t stream);

/* As rtopk_maxk_forward with one-byte indices. Requires M <= 256. */
rtopk_status_t rtopk_maxk_forward_u8(const float* x, int64_t N, int32_t M,
                                     int32_t k, float* y, float* sp_data,
                                     uint8_t* sp_index, hipStream_t stream);

/*
 * MaxK backward (MaxK-GNN review, "How MaxK-GNN works": only the survivors of
 * the MaxK nonlinearity carry gradient, and the backward pass reuses the
 * sp_index the forward pass produced). Writes the dense [N, M] gradient
 *   grad_x[r*M + sp_index[r*k + i]] = grad_sp[r*k + i]   for i < k,
 * and +0.0 in every column no entry of row r names. The same call turns a
 * compressed row pair (sp_data, sp_index) back into the dense MaxK output.
 *   grad_sp   device pointer to N*k floats (gradient of the survivors, in
 *             the order of sp_index), read.
 *   sp_index  device pointer to N*k int32 column indices, read. The indices
 *             of a row must be distinct for the result to be defined (MaxK's
 *             are); with duplicates one of the entries lands, unspecified
 *             which. Entries outside [0, M) are ignored.
 *   grad_x    device pointer to N*M floats, written (every element).
 * N, M, k, stream and the errors are as above (1 <= k <= M <= 8192).
 * grad_x must not overlap the inputs.
 */
rtopk_status_t rtopk_maxk_backward(const float* grad_sp,
                                   const int32_t* sp_index, int64_t N,
                                   int32_t M, int32_t k, float* grad_x,
                                   hipStream_t stream);

/* As rtopk_maxk_backward with one-byte indices. Requires M <= 256. */
rtopk_status_t rtopk_maxk_backward_u8(const float* grad_sp,
                                      const uint8_t* sp_index, int64_t N,
                                      int32_t M, int32_t k, float* grad_x,
                                      hipStream_t stream);

/*
 * MaxK-GNN forward aggregation (MaxK-GNN review, "How MaxK-GNN works": a
 * row-wise product SpGEMM over the compressed features, each output row
 * accumulated on chip and written once; abstract: CBSR feature fetching and
 * a shared-memory accumulation buffer). Computes the dense
 *   y[i*M + c] = sum over e in [row_ptr[i], row_ptr[i+1]) and t < k with
 *                sp_index[col_idx[e]*k + t] == c of val[e] * sp_data[col_idx[e]*k + t]
 * in single precision (fused multiply-adds in an unspecified order:
 * the result differs from the exact sum by at most (d + 1) * 2^-24 times the
 * sum of the terms' magnitudes, d the number of terms; rows cut between two
 * work ranges are summed with atomics, so repeated calls may differ in the
 * last bits).
 *   row_ptr   device pointer to n_dst + 1 int64: the CSR row offsets of A,
 *             nondecreasing, row_ptr[0] == 0, row_ptr[n_dst] == nnz.
 *   col_idx   device pointer to nnz int32 source rows in [0, n_src).
 *   val       device pointer to nnz floats: the edge weights.
 *   n_dst     rows of A and of y (>= 0); n_src rows of the compressed
 *             features (>= 1 when nnz > 0); nnz edges (>= 0).
 *   sp_data, sp_index  the compressed features, [n_src, k] floats and
 *             int32 (uint8 for the _u8 form) columns in [0, M), distinct
 *             within a row, as written by rtopk_select_exact or
 *             rtopk_maxk_forward (with repeated columns in a row the result
 *             is unspecified).
 *   M, k      feature width and survivors per row, 1 <= k <= M <= 8192.
 *   y         device pointer to n_dst * M floats, written (every element).
 * Edges whose column lies outside [0, n_src) and survivors whose column lies
 * outside [0, M) contribute nothing. With row_ptr breaking its conditions
 * the result is unspecified, but every access stays inside the arrays. Two
 * kernels are enqueued on `stream` (rows cut between ranges are zeroed
 * first). Errors as above, plus RTOPK_ERROR_INVALID_VALUE for nnz < 0,
 * n_src < 0, or n_src == 0 with nnz > 0.
 */
rtopk_status_t rtopk_cbsr_spgemm(const int64_t* row_ptr, const int32_t* col_idx,
                                 const float* val, int64_t n_dst, int64_t n_src,
                                 int64_t nnz, const float* sp_data,
                                 const int32_t* sp_index, int32_t M, int32_t k,
                                 float* y, hipStream_t stream);

/* As rtopk_cbsr_spgemm with one-byte survivor columns. Requires M <= 256. */
rtopk_status_t rtopk_cbsr_spgemm_u8(const int64_t* row_ptr, const int32_t* col_idx,
                                    const float* val, int64_t n_dst, int64_t n_src,
                                    int64_t nnz, const float* sp_data,
                                    const uint8_t* sp_index, int32_t M, int32_t k,
                                    float* y, hipStream_t stream);

/*
 * Backward of rtopk_cbsr_spgemm with respect to the compressed features
 * (MaxK-GNN review, "How MaxK-GNN works": the backward samples exactly the
 * sp_index positions, reusing the forward's sparsity pattern, with an
 * outer-product dataflow and dense-row prefetching). Given the gradient dy
 * of y, computes
 *   grad_sp[j*k + t] = sum over edges e = (i -> j), i.e. e in
 *                      [row_ptr[i], row_ptr[i+1]) with col_idx[e] == j, of
 *                      val[e] * dy[i*M + sp_index[j*k + t]]
 * (A^T dy sampled at the survivors), in single precision with float
 * atomics: the order of the sums is unspecified and repeated calls may
 * differ in the last bits (bound as for rtopk_cbsr_spgemm, d the number of
 * edges into j).
 *   row_ptr, col_idx, val, n_dst, n_src, nnz  the same CSR of A as the
 *             forward (no transpose needed).
 *   dy        device pointer to n_dst * M floats, read.
 *   sp_index  device pointer to n_src * k int32 (uint8 for the _u8 form)
 *             columns in [0, M), read.
 *   grad_sp   device pointer to n_src * k floats, written (every element;
 *             survivors with no edge get +0.0).
 * Edges whose column lies outside [0, n_src) and survivors outside [0, M)
 * contribute nothing. Two kernels are enqueued on `stream`. Errors as for
 * rtopk_cbsr_spgemm (grad_sp may not be NULL when n_src > 0).
 */
rtopk_status_t rtopk_cbsr_sspmm(const int64_t* row_ptr, const int32_t* col_idx,
                                const float* val, int64_t n_dst, int64_t n_src,
                                int64_t nnz, const float* dy,
                                const int32_t* sp_index, int32_t M, int32_t k,
                                float* grad_sp, hipStream_t stream);

/* As rtopk_cbsr_sspmm with one-byte survivor columns. Requires M <= 256. */
rtopk_status_t rtopk_cbsr_sspmm_u8(const int64_t* row_ptr, const int32_t* col_idx,
                                   const float* val, int64_t n_dst, int64_t n_src,
                                   int64_t nnz, const float* dy,
                                   const uint8_t* sp_index, int32_t M, int32_t k,
                                   float* grad_sp, hipStream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* rtopk_status_string(rtopk_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* RTOPK_H_ */
