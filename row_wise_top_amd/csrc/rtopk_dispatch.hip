// Host-side dispatch of the row kernels: picks the kernel for the row length,
// sizes a persistent grid to the device's resident capacity, and enqueues it.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <mutex>
#include <unordered_map>

#include "rtopk_internal.h"

namespace rtopk {

// Resident blocks per CU for a kernel on a device, cached per device.
int resident_blocks(const void* fn, int threads, int device) {
  static std::mutex mu;
  static std::unordered_map<const void*, int> cache[64];
  std::lock_guard<std::mutex> lock(mu);
  auto& c = cache[device & 63];
  auto it = c.find(fn);
  if (it != c.end()) return it->second;
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, fn, threads, 0) !=
          hipSuccess ||
      blocks < 1)
    blocks = 1;
  c.emplace(fn, blocks);
  return blocks;
}

int cu_count(int device) {
  static std::mutex mu;
  static int cached[64] = {0};
  std::lock_guard<std::mutex> lock(mu);
  int& c = cached[device & 63];
  if (c == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount,
                              device) != hipSuccess ||
        v < 1)
      v = 1;
    c = v;
  }
  return c;
}

namespace {


int slot_bucket(int m) {
  const int slots = (m + kWave - 1) / kWave;
  for (int b : kSlotBuckets) {
    if (b >= slots) return b;
  }
  return 0;
}

RowsKernel kernel_for(int m, Mode mode, bool u8_index, int qc) {
  const int q = slot_bucket(m);
  const bool full = (m == q * kWave);
  switch (q) {
    case 1: return rows_kernel<1>(full, mode, u8_index, qc);
    case 2: return rows_kernel<2>(full, mode, u8_index, qc);
    case 3: return rows_kernel<3>(full, mode, u8_index, qc);
    case 4: return rows_kernel<4>(full, mode, u8_index, qc);
    case 6: return rows_kernel<6>(full, mode, u8_index, qc);
    case 8: return rows_kernel<8>(full, mode, u8_index, qc);
    case 12: return rows_kernel<12>(full, mode, u8_index, qc);
    case 16: return rows_kernel<16>(full, mode, u8_index, qc);
    case 24: return rows_kernel<24>(full, mode, u8_index, qc);
    case 32: return rows_kernel<32>(full, mode, u8_index, qc);
    case 48: return rows_kernel<48>(full, mode, u8_index, qc);
    case 64: return rows_kernel<64>(full, mode, u8_index, qc);
    case 96: return rows_kernel<96>(full, mode, u8_index, qc);
    case 128: return rows_kernel<128>(full, mode, u8_index, qc);
    default: return nullptr;
  }
}

// Upper-tail quantile of the standard normal: z with P(Z > z) = p.
double normal_upper_quantile(double p) {
  double lo = -9.0, hi = 9.0;
  for (int i = 0; i < 80; ++i) {
    const double mid = 0.5 * (lo + hi);
    if (0.5 * std::erfc(mid / std::sqrt(2.0)) > p)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

double normal_density(double z) {
  return std::exp(-0.5 * z * z) / std::sqrt(2.0 * 3.14159265358979323846);
}

// Normal-model steering of the exact search (see rtopk_rows.hpp): the first
// threshold aims at the middle of (k, 64*qc] elements (or k + 1/2 without
// compaction); Newton steps use the density at the k-th largest value.
void exact_model(SelectArgs& a, int qc) {
  // The constants depend on (m, k, qc) only, and two quantiles take 160
  // erfc evaluations (~4.4 us of host time): each thread keeps the last set.
  struct Model {
    int m = -1, k = -1, qc = -1;
    float z_first, half_step, z_first_c, half_step_c, inv_m;
  };
  thread_local Model last;
  if (last.m == a.m && last.k == a.k && last.qc == qc) {
    a.z_first = last.z_first;
    a.half_step = last.half_step;
    a.z_first_c = last.z_first_c;
    a.half_step_c = last.half_step_c;
    a.inv_m = last.inv_m;
    return;
  }
  const double m = a.m;
  const double clamp_lo = 0.5 / m, clamp_hi = 1.0 - 0.5 / m;
  auto frac = [&](double count) {
    return std::fmin(std::fmax(count / m, clamp_lo), clamp_hi);
  };
  const double first = qc > 0 ? 0.5 * (a.k + kWave * qc) : a.k + 0.5;
  const double z_first = normal_upper_quantile(frac(first));
  const double z_k = normal_upper_quantile(frac(a.k + 0.5));
  // The kernel has r = sqrt(sum x^2) = rms * sqrt(m); fold 1/sqrt(m) in.
  const double inv_sqrt_m = 1.0 / std::sqrt(m);
  a.z_first = static_cast<float>(z_first * inv_sqrt_m);
  a.half_step = static_cast<float>(0.5 / (m * normal_density(z_k)) * inv_sqrt_m);
  a.z_first_c = static_cast<float>(z_first);
  a.half_step_c = static_cast<float>(0.5 / (m * normal_density(z_k)));
  a.inv_m = static_cast<float>(1.0 / m);
  last = Model{a.m, a.k, qc, a.z_first, a.half_step, a.z_first_c, a.half_step_c, a.inv_m};
}

// Exact or capped search on rows longer than kGroupMinLength: one row per
// block of four waves (rtopk_group.hpp), on a persistent grid of what fits
// on the device at once.
hipError_t launch_group(const SelectArgs& a, int qc, bool capped, hipStream_t stream) {
  constexpr int kPerSlot = kWave * kWavesPerRowGroup;
  const int per_wave = (a.m + kPerSlot - 1) / kPerSlot;
  const int q = per_wave <= 24 ? 24 : 32;
  const bool full = a.m == q * kPerSlot;
  const RowsKernel fn = q == 24 ? group_kernel<24>(full, false, qc, capped)
                                : group_kernel<32>(full, false, qc, capped);
  if (fn == nullptr) return hipErrorInvalidValue;
  int device = 0;
  hipError_t err = hipGetDevice(&device);
  if (err != hipSuccess) return err;
  const int threads = kWave * kWavesPerRowGroup;
  const int64_t resident =
      static_cast<int64_t>(cu_count(device)) *
      resident_blocks(reinterpret_cast<const void*>(fn), threads, device);
  const int64_t grid = a.n < resident ? a.n : resident;
  hipLaunchKernelGGL(fn, dim3(static_cast<uint32_t>(grid)), dim3(threads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const SelectArgs& args, Mode mode, bool u8_index,
                         hipStream_t stream) {
  SelectArgs a = args;
  // The capped search with no cap and eps = 0 ends exactly where the exact
  // search does (a count of k, or lo and hi adjacent floats with lo the k-th
  // largest value; the tie fill then takes the lowest columns holding it),
  // so the exact kernel computes it.
  if (mode == Mode::kCapped && a.max_iter < 0 && a.eps == 0.0f) mode = Mode::kExact;
  // Candidate slots: the exact search compacts after its first count; the
  // capped search stages at the same model threshold (capped_row).
  const int q = slot_bucket(a.m);
  const int qc = mode == Mode::kCapped ? capped_candidate_slots(q, a.k, a.max_iter)
                                       : exact_candidate_slots(q, a.k);
  if (mode != Mode::kCapped || qc > 0) exact_model(a, qc);
  // Row groups: exact search above 4,096 columns; capped search above
  // 6,144 (at 6,000 columns one wave per row was faster: 76.6 against
  // 101.6 us for 16,384 rows with few distinct values, k = 64, 4 steps).
  if (!u8_index && ((mode == Mode::kExact && a.m > kGroupMinLength) ||
                    (mode == Mode::kCapped && a.m > kCappedGroupMinLength)))
    return launch_group(a, qc, mode == Mode::kCapped, stream);
  const RowsKernel fn = kernel_for(a.m, mode, u8_index, qc);
  if (fn == nullptr) return hipErrorInvalidValue;
  int device = 0;
  hipError_t err = hipGetDevice(&device);
  if (err != hipSuccess) return err;
  // One wave per row at a time, in groups of D = rows_in_flight(q, .) rows.
  // Short rows: one group per wave, a grid over the whole matrix (waves exit
  // after their group). Long rows: a persistent grid of what fits on the
  // device at once.
  const int64_t d = rows_in_flight(q, mode == Mode::kMaxk);
  const int threads = kWave * row_waves(q);
  const int64_t per_block = row_waves(q) * d;
  const int64_t blocks_needed = (a.n + per_block - 1) / per_block;
  int64_t grid = blocks_needed;
  if (!one_group_per_wave(q) || blocks_needed > 0x7fffffff) {
    const int64_t resident =
        static_cast<int64_t>(cu_count(device)) *
        resident_blocks(reinterpret_cast<const void*>(fn), threads, device);
    grid = blocks_needed < resident ? blocks_needed : resident;
  }
  hipLaunchKernelGGL(fn, dim3(static_cast<uint32_t>(grid)), dim3(threads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace rtopk
