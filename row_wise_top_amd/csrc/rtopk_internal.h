// Internal interface between the C ABI (rtopk_api.hip) and the kernels
// (rtopk_dispatch.hip and the rtopk_*.hip units it names). Not installed; not
// part of the public ABI.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace rtopk {

// Largest row length the one-wave-per-row kernels hold in registers.
constexpr int kMaxRowLength = 8192;
constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWave * kWavesPerBlock;
// Waves per block of the one-wave-per-row selection kernels, by slots per
// lane q: single-wave blocks for rows of at most 512 columns (a wave's slot
// on the CU frees as soon as it ends, not when the slowest of its block
// does), four waves for longer rows.
constexpr int row_waves(int q) { return q <= 8 ? 1 : 4; }

// Waves that share one row in the row-group kernel (rtopk_group.hpp), used
// by the exact search for rows longer than kGroupMinLength and by the
// capped search for rows longer than kCappedGroupMinLength.
constexpr int kWavesPerRowGroup = 4;
constexpr int kGroupMinLength = 4096;        // exact search: longer rows
constexpr int kCappedGroupMinLength = 6144;  // capped search: longer rows

// kMaxk: the exact search, plus the dense [n, m] MaxK output (SelectArgs::dense).
// kBucket: the exact search on buckets: each kernel row is one bucket of an
// input row (SelectArgs::buckets of them, m columns each) and emitted
// columns are offset by the bucket's position in its row.
enum class Mode { kCapped, kExact, kMaxk, kBucket };

struct SelectArgs {
  const float* x;
  int64_t n;
  int32_t m;
  int32_t k;
  int32_t max_iter;  // capped mode only; < 0 = no cap
  float eps;         // capped mode only; >= 0
  float* out_val;
  void* out_idx;     // int32_t* or uint8_t*
  // Exact search only: thresholds from a normal model of the row (host
  // computed; they steer the search, never its result).
  // With r = sqrt(sum of squares of the row) = rms * sqrt(m):
  float z_first;     // first threshold = r * z_first
  float half_step;   // Newton step per doubled count = r * half_step
  float* dense;      // Mode::kMaxk only: [n, m] output, survivors kept, rest 0
  int32_t buckets;   // Mode::kBucket only: buckets per input row (>= 1)
  // Exact search, second try for rows whose first count misses: the same
  // model on the row's mean and standard deviation sd.
  float z_first_c;   // threshold = mean + sd * z_first_c
  float half_step_c; // Newton step per doubled count = sd * half_step_c
  float inv_m;       // 1 / m
};

using RowsKernel = void (*)(SelectArgs);

// Rows a wave of the selection kernel keeps in flight for q slots per lane:
// the row being worked on plus rows_in_flight(q, dense) - 1 whose loads are
// issued. About 4 KB of a wave's rows are in flight for rows of at most 384
// columns, two rows of 385 to 512; the fused MaxK forward (dense: it also
// writes each row back whole) keeps two. From 513 columns one row per wave:
// a second row's search then waited behind the first's (one box, us, two
// rows -> one: 1,048,576 x 1,024 N(0,1), k = 64 820 -> 771, capped with 4
// steps 834 -> 765; 16,384 x 1,024 rows with ties, k = 128 21.9 -> 18.5;
// 262,144 x 768, k = 64 151 -> 144; at 512 columns one row per wave was
// 6% slower on N(0,1) rows). Short rows (q <= 16) are also the rows each
// wave takes in all: the grid then covers the matrix once (a wave that
// loads its rows first and stores last never waits on its own stores,
// which share the load counter on this GPU). Longer rows get no prefetch.
constexpr int rows_in_flight(int q, bool dense) {
  return q > 16 ? 1 : dense ? 2 : q <= 2 ? 8 : q <= 6 ? 4 : q <= 8 ? 2 : 1;
}
// Rows of up to 2,048 columns: one group per wave over the whole matrix;
// the hardware's dispatcher then balances the waves, where a persistent
// grid's equal shares waited for its slowest waves (one box, us, persistent
// -> one group per wave: 65,536 x 2,048 N(0,1), k = 64 108.6 -> 92.2;
// 16,384 x 2,048 tie-heavy rows, k = 32 28.9 -> 26.3, k = 256 32.7 -> 31.0;
// at 4,096 columns the persistent grid stays ahead, 197.1 against 205.8 on
// 65,536 N(0,1) rows).
constexpr bool one_group_per_wave(int q) { return q <= 32; }

// Rows the fused MaxK forward kernel takes (its LDS holds the dense row);
// longer rows run the selection and then the scatter.
constexpr bool maxk_fused(int q) { return q <= 16; }

// Bucket lengths the bucketed kernels take (64*q columns, q <= 16).
constexpr bool bucket_supported(int q) { return q <= 16; }

// Slot counts Q (elements per lane) with an instantiated register-resident
// row kernel; a row of length m uses the smallest Q with 64*Q >= m.
constexpr int kSlotBuckets[] = {1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 48, 64, 96, 128};

// Defined in rtopk_rows.hpp, instantiated in the rtopk_rows_*.hip units.
// qc: candidate slots of the exact search (0: no compaction).
template <int Q>
RowsKernel rows_kernel(bool full, Mode mode, bool u8_index, int qc);

// Defined in rtopk_group.hpp, instantiated in rtopk_group.hip: the exact
// (or capped) kernel for rows held by a group of four waves, q slots per lane
// per wave.
template <int Q>
RowsKernel group_kernel(bool full, bool u8_index, int qc, bool capped);

// Candidate slots QC the exact search compacts into for q slots and k
// survivors: the smallest of 1, 2, 4, 8 with 64*QC >= 2k and 2*QC <= q, or 0
// when there is none (the search then stays on the whole row).
inline int candidate_slots(int q, int k) {
  for (int qc : {1, 2, 4, 8}) {
    if (kWave * qc >= 2 * k && 2 * qc <= q) return qc;
  }
  return 0;
}

// Candidate slots of the exact search: rows of 1,024 columns and more take
// a window of 4k candidates where one is built, shorter rows one of 2k
// (candidate_slots). The wider window lets more first counts land in it;
// rows with many equal values gain most, since their counts jump in large
// steps. Measured (one box, 2k against 4k window, us): 16,384 rows of
// N(0,1) rounded to steps of 0.25, k = 64, at 1,024 / 2,048 / 4,096 / 8,192
// columns: 19.0 / 17.8, 35.8 / 27.7, 70.2 / 52.2, 207 / 139.5; N(0,1)
// rows: 1,048,576 x 1,024, k = 64, 831 / 824; 262,144 x 1,024, k = 32,
// 190.6 / 187.8; 65,536 x 2,048, k = 64, 107.1 / 111.1. At 256 and 512
// columns the 4k window was slower (headline 56.0 against 63.1).
inline int exact_candidate_slots(int q, int k) {
  if (q >= 16) {
    for (int qc : {1, 2, 4, 8}) {
      if (kWave * qc >= 4 * k && 2 * qc <= q) return qc;
    }
  }
  return candidate_slots(q, k);
}

// Candidate slots of the capped search (see capped_row): the capped kernel
// stages the elements above the exact search's first threshold (steered by
// the exact search's model constants for this window) before its first
// step, and every step then compares the candidate slots. Up to four steps,
// and rows of 4,096 columns or more: the exact search's window (wider for
// long rows, so that more first counts land in it); more steps on shorter
// rows, or no cap: the 2k window, whose steps compare fewer slots. Measured
// (one box, us, 2k window against the exact one): 1,048,576 x 1,024 N(0,1),
// k = 64, 8 steps 829.5 / 826.1; 262,144 x 1,024, k = 32, 6 steps 189.0 /
// 193.1; 16,384 rows of N(0,1) rounded to steps of 0.25 (ties), 6 steps,
// k = 64: 2,048 columns 29.0 / 30.0, 4,096 columns 63.5 / 54.7, 8,192
// columns 222.9 / 138.3; 8,192 columns, k = 32, 5 steps 253.1 / 130.8;
// 65,536 x 8,192 N(0,1), k = 64, 6 steps 501.8 / 514.4. A search with no
// cap and eps = 0 never reaches this: its result is the canonical exact
// top-k, and launch_select runs the exact kernel for it. At most two
// steps on rows of up to 512 columns: no candidates (the steps and the tie
// fill count over the row, whose output is assembled in LDS); staging costs
// more than the two counts it saves (262,144 x 256, k = 32, 2 steps 55.6 ->
// 54.0 us; 65,536 x 256, k = 32 19.0 -> 18.9 us; with 3 steps staging wins:
// 57.6 against 58.6 us).
inline int capped_candidate_slots(int q, int k, int max_iter) {
  if (max_iter >= 0 && max_iter <= 2 && q <= 8) return 0;
  if ((max_iter >= 0 && max_iter <= 4) || q >= 64) return exact_candidate_slots(q, k);
  return candidate_slots(q, k);
}

// Resident blocks per CU of `fn` launched with `threads` threads per block on
// `device`, and the device's CU count (both cached per device).
int resident_blocks(const void* fn, int threads, int device);
int cu_count(int device);

// MaxK backward (and compressed rows to dense): out[r, idx[r, i]] = src[r, i]
// for every entry with an index in [0, m), every other element of out 0.
struct ScatterArgs {
  const float* src;  // [n, k]
  const void* idx;   // [n, k] int32_t or uint8_t
  int64_t n;
  int32_t m;
  int32_t k;
  float* out;        // [n, m]
};

// Enqueue the scatter kernel (rtopk_maxk.hip). Arguments are validated
// (n > 0, 1 <= k <= m <= kMaxRowLength).
hipError_t launch_scatter(const ScatterArgs& a, bool u8_index,
                          hipStream_t stream);

// MaxK-GNN forward aggregation Y = A X (rtopk_spgemm.hip): A in CSR, X as
// compressed rows (sp_data, sp_index: k survivors of m columns per row).
struct SpgemmArgs {
  const int64_t* row_ptr;  // [n_dst + 1]
  const int32_t* col;      // [nnz], source rows
  const float* val;        // [nnz]
  int64_t n_dst;
  int64_t n_src;           // >= 1
  int64_t nnz;
  const float* sp_data;    // [n_src, k]
  const void* sp_index;    // [n_src, k] int32_t or uint8_t
  int32_t m;
  int32_t k;
  float* y;                // [n_dst, m]
  // Set by launch_spgemm.
  int64_t chunk;           // edges per wave
  int64_t waves;           // waves of the main kernel
  int32_t m_pad;           // LDS floats per wave
  int32_t waves_per_block; // 1 to kWavesPerBlock
  int32_t slots;           // edges per step (accumulator rows per wave)
};

// Edges each wave of the aggregation takes.
constexpr int64_t kEdgesPerWave = 256;

// Enqueue the aggregation (a zeroing kernel for rows cut by a wave's range,
// then the main kernel). Arguments validated (n_dst >= 0, n_src >= 1 when
// nnz > 0, 1 <= k <= m <= kMaxRowLength).
hipError_t launch_spgemm(SpgemmArgs a, bool u8_index, hipStream_t stream);

// Enqueue the backward of the aggregation to the compressed features
// (rtopk_spgemm.hip), with the same SpgemmArgs read as: sp_data = dY
// ([n_dst, m]), sp_index the survivors' columns ([n_src, k]), y = grad_sp
// ([n_src, k], zeroed, then accumulated).
hipError_t launch_sspmm(SpgemmArgs a, bool u8_index, hipStream_t stream);

// Bucketed top-k with short buckets (rtopk_bucket.hip): one lane per bucket
// for buckets of at most kLaneBucketWidth columns keeping at most
// kLaneBucketSurvivors each; four lanes per bucket for buckets of up to
// kQuadBucketWidth columns keeping at most kQuadBucketSurvivors, where the
// width is a multiple of 4 and x is 16-byte aligned. `a` is the bucket view
// (n = rows * buckets, m = bucket width, k = survivors per bucket, buckets
// = buckets per row).
constexpr int kLaneBucketWidth = 64;
constexpr int kLaneBucketSurvivors = 8;
constexpr int kQuadBucketWidth = 128;
constexpr int kQuadBucketSurvivors = 16;
bool bucket_lanes_supported(const float* x, int width, int kb);
hipError_t launch_bucket_lanes(const SelectArgs& a, bool u8_index,
                               hipStream_t stream);

// Enqueue the selection kernel for `a` on `stream`. Arguments are already
// validated (1 <= k <= m <= kMaxRowLength, n > 0, u8 only with m <= 256).
// Returns the HIP error of the launch.
hipError_t launch_select(const SelectArgs& a, Mode mode, bool u8_index,
                         hipStream_t stream);

}  // namespace rtopk
