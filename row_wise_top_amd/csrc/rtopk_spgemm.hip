// MaxK-GNN forward aggregation on gfx950: Y = A X with A a CSR graph and X
// given by its compressed MaxK rows (k survivors of M columns: sp_data,
// sp_index). MaxK-GNN review, "How MaxK-GNN works": a row-wise product
// SpGEMM that accumulates each output row on chip and writes it to global
// memory once; the abstract names the compressed balanced layout for the
// feature fetches and a shared-memory accumulation buffer.
//
// Work split. Power-law graphs have rows thousands of edges long, so rows
// are not the unit of work: wave w takes edges [w*C, (w+1)*C) of the CSR
// arrays (C = kEdgesPerWave) and every row that starts there, plus the part
// of the row that was cut at its first edge. Each row (or part of a row) is
// accumulated in the wave's own LDS rows (one lane per (edge, survivor)
// pair, up to 4 edges per instruction, see accumulate), then flushed:
//  * a row wholly inside the wave's range is stored once;
//  * a row cut by a range boundary is added to Y with float atomics; such
//    rows are zeroed first by a small kernel (one lane per row).
// Every wave does about the same number of edges whatever the degree
// distribution, and each complete row still reaches HBM exactly once.
//
// Inputs that break the preconditions (row_ptr not nondecreasing, indices
// out of range) give an unspecified result but no out-of-bounds access:
// every read is clamped into its array and out-of-range columns and
// indices are skipped.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rtopk_internal.h"

namespace rtopk {
namespace spgemm_detail {

constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ uint64_t ballot(bool p) {
  return __builtin_amdgcn_ballot_w64(p);
}

// Largest i in [0, n] with row_ptr[i] <= p, by a 64-way search (each step
// samples 64 positions, one per lane). row_ptr[0] <= p is assumed; with a
// row_ptr that is not nondecreasing the result is some i in [0, n].
__device__ int64_t last_row_at_or_before(const int64_t* __restrict__ row_ptr,
                                         int64_t n, int64_t p, int lane) {
  int64_t lo = 0, hi = n;
  while (hi > lo) {
    const int64_t step = (hi - lo + 63) / 64;
    const int64_t q = lo + (lane + 1) * step;
    const bool le = q <= hi && row_ptr[q <= hi ? q : hi] <= p;
    const int cnt = __popcll(ballot(le));
    const int64_t new_hi = lo + (cnt + 1) * step - 1;
    lo = lo + cnt * step;
    hi = new_hi < hi ? new_hi : hi;
  }
  return lo;
}

// Clamp a row_ptr entry into [0, nnz].
__device__ __forceinline__ int64_t clamp_edge(int64_t e, int64_t nnz) {
  return e < 0 ? 0 : (e > nnz ? nnz : e);
}

// Zero Y[i, :] for every row i cut by an interior range boundary
// p = w * C (w >= 1): start < p < end. The smallest multiple of C above
// start is (start / C + 1) * C, so the row is cut iff that lies below end.
// One lane per row reads its two offsets (coalesced), then the wave clears
// its cut rows one after another. A hub row that many boundaries cut is
// cleared once (one wave per boundary, each first searching row_ptr for its
// row, took 23 us on the 262,144-node graph).
__global__ __launch_bounds__(kBlock) void zero_cut_rows(SpgemmArgs a) {
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  const int64_t base =
      static_cast<int64_t>(blockIdx.x) * kBlock +
      __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave) * kWave;
  const int64_t i = base + lane;
  bool cut = false;
  if (i < a.n_dst) {
    const int64_t start = clamp_edge(a.row_ptr[i], a.nnz);
    const int64_t end = clamp_edge(a.row_ptr[i + 1], a.nnz);
    cut = (start / a.chunk + 1) * a.chunk < end;
  }
  for (uint64_t mask = ballot(cut); mask != 0; mask &= mask - 1) {
    const int64_t r = base + __builtin_ctzll(mask);
    const __amdgpu_buffer_rsrc_t ry =
        __builtin_amdgcn_make_buffer_rsrc(a.y + r * a.m, 0, a.m * 4, kRsrcWord3);
    for (int c = lane; c < a.m; c += kWave)
      __builtin_amdgcn_raw_buffer_store_b32(0u, ry, c * 4, 0, 0);
  }
}

// Accumulate edges [s0, s1) of a row into the wave's LDS accumulators. The
// edges' source rows and weights come from the wave's LDS copy of its edge
// range (ecol / eval, indexed from the range's first edge e0), so the only
// global loads in the loop are the features, issued for U steps at a time.
//
// Lane roles: a step takes P edges (P = min(4, 64 / k) for k <= 64, else 1);
// lane l serves edge slot l / k and survivor l % k (lanes past P*k idle;
// for k > 64 each edge takes ceil(k / 64) passes). Each edge slot adds into
// its own accumulator row (accp), with a plain read, fma and write: the
// survivors of one edge have distinct columns and the slots never share a
// row, so no two lanes of an instruction touch one word, and the LDS
// pipeline applies one wave's instructions in order. (LDS float atomics
// would serialise about one lane per clock.)
template <typename IdxT>
__device__ __forceinline__ void accumulate(const SpgemmArgs& a, int64_t e0,
                                           int64_t s0, int64_t s1, float* accp,
                                           const int* ecol, const float* eval,
                                           int lane_edge, int lane_t, int P) {
  const IdxT* sidx = static_cast<const IdxT*>(a.sp_index);
  const int k = a.k;
  // Idle lanes (lane_edge < 0) address the step's first edge and add nothing.
  const int addr_edge = lane_edge < 0 ? 0 : lane_edge;
  // Steps whose feature loads are issued together (measured on the
  // 262,144-node graph, without the pipelining below: four steps 582 us at
  // 8 waves per SIMD, eight 626 us at 5).
  constexpr int U = 4;
  // One survivor per lane (k <= 64): the next U steps' feature loads are
  // issued before the current ones are added, so each wave keeps loads in
  // flight while it works on the LDS accumulators (569 -> 561 us; two or
  // three steps per batch measured the same).
  if (k <= kWave) {
    struct Step {
      float xv[U], w[U];
      int xc[U];
      bool ok[U];
    };
    auto load = [&](int64_t b0, Step& st) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t e = b0 + static_cast<int64_t>(u) * P + addr_edge;
        const int64_t ec = e < s1 ? e : s1 - 1;  // stays inside the staged range
        const int col = ecol[ec - e0];
        st.w[u] = eval[ec - e0];
        const bool live = lane_edge >= 0 && e < s1 &&
                          static_cast<uint64_t>(static_cast<int64_t>(col)) <
                              static_cast<uint64_t>(a.n_src);
        const int64_t j = live ? col : 0;
        st.xv[u] = a.sp_data[j * k + lane_t];
        st.xc[u] = static_cast<int>(sidx[j * k + lane_t]);
        st.ok[u] = live;
      }
    };
    Step cur, nxt;
    if (s0 < s1) load(s0, cur);
    for (int64_t b0 = s0; b0 < s1; b0 += static_cast<int64_t>(U) * P) {
      const int64_t b1 = b0 + static_cast<int64_t>(U) * P;
      if (b1 < s1) load(b1, nxt);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (cur.ok[u] && static_cast<uint32_t>(cur.xc[u]) < static_cast<uint32_t>(a.m))
          accp[cur.xc[u]] = fmaf(cur.w[u], cur.xv[u], accp[cur.xc[u]]);
      }
      cur = nxt;
    }
    return;
  }
  for (int64_t b0 = s0; b0 < s1; b0 += static_cast<int64_t>(U) * P) {
    for (int t0 = lane_t; t0 < k; t0 += kWave) {
      float xv[U], w[U];
      int xc[U];
      bool ok[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t e = b0 + static_cast<int64_t>(u) * P + addr_edge;
        const int64_t ec = e < s1 ? e : s1 - 1;  // stays inside the staged range
        const int col = ecol[ec - e0];
        w[u] = eval[ec - e0];
        const bool live = lane_edge >= 0 && e < s1 &&
                          static_cast<uint64_t>(static_cast<int64_t>(col)) <
                              static_cast<uint64_t>(a.n_src);
        const int64_t j = live ? col : 0;
        xv[u] = a.sp_data[j * k + t0];
        xc[u] = static_cast<int>(sidx[j * k + t0]);
        ok[u] = live;
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (ok[u] && static_cast<uint32_t>(xc[u]) < static_cast<uint32_t>(a.m))
          accp[xc[u]] = fmaf(w[u], xv[u], accp[xc[u]]);
      }
      if (k <= kWave) break;  // one pass covers the survivors
    }
  }
}

// Store (or, for a cut row, add) the sum of the wave's P accumulator rows to
// Y[i, :], then zero them.
__device__ __forceinline__ void flush(const SpgemmArgs& a, int64_t i, float* acc,
                                      int P, int lane, bool cut) {
  __builtin_amdgcn_wave_barrier();
  const __amdgpu_buffer_rsrc_t ry =
      __builtin_amdgcn_make_buffer_rsrc(a.y + i * a.m, 0, a.m * 4, kRsrcWord3);
  for (int c = lane; c < a.m; c += kWave) {
    float v = acc[c];
    acc[c] = 0.0f;
    for (int p = 1; p < P; ++p) {
      v += acc[p * a.m_pad + c];
      acc[p * a.m_pad + c] = 0.0f;
    }
    if (cut)
      unsafeAtomicAdd(a.y + i * a.m + c, v);  // hardware float atomic
    else
      // Non-temporal (gfx950 cache policy bit 1): y is written once.
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), ry, c * 4, 0, 2);
  }
  __builtin_amdgcn_wave_barrier();
}

// Blocks of a.waves_per_block waves (fewer for long rows, so that a block's
// LDS rows stay within 64 KB).
template <typename IdxT>
__global__ __launch_bounds__(kBlock) void spgemm_rows(SpgemmArgs a) {
  extern __shared__ float lds[];
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  const int wave_in_block =
      __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  // Per wave: P accumulator rows (m_pad floats each), then the staged edge
  // range (kEdgesPerWave source rows, kEdgesPerWave weights).
  const int P = a.slots;
  float* acc = lds + static_cast<int64_t>(wave_in_block) * (P * a.m_pad + 2 * kEdgesPerWave);
  int* ecol = reinterpret_cast<int*>(acc + P * a.m_pad);
  float* eval = acc + P * a.m_pad + kEdgesPerWave;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * a.waves_per_block + wave_in_block;
  if (w >= a.waves) return;
  const int64_t nnz = a.nnz;
  const int64_t e0 = w * a.chunk;
  const int64_t e1 = e0 + a.chunk < nnz ? e0 + a.chunk : nnz;
  const bool last = w == a.waves - 1;
  // Stage the range's edges (coalesced; positions past e1 re-read e1 - 1).
  for (int j = lane; j < kEdgesPerWave; j += kWave) {
    const int64_t e = e0 + j < e1 ? e0 + j : e1 - 1;
    // The CSR arrays are read once: non-temporal loads.
    ecol[j] = e >= 0 ? __builtin_nontemporal_load(a.col + e) : 0;
    eval[j] = e >= 0 ? __builtin_nontemporal_load(a.val + e) : 0.0f;
  }
  // LDS operations of one wave complete in issue order; the barrier keeps
  // the compiler from moving the reads below above these writes.
  __builtin_amdgcn_wave_barrier();
  // Lane roles: edge slot within a step and survivor index.
  const int k = a.k;
  const int lane_edge = k <= kWave ? (lane < P * k ? lane / k : -1) : 0;
  const int lane_t = k <= kWave ? lane % k : lane;
  float* accp = acc + (lane_edge > 0 ? lane_edge : 0) * a.m_pad;
  for (int c = lane; c < P * a.m_pad; c += kWave) acc[c] = 0.0f;
  __builtin_amdgcn_wave_barrier();
  // The row cut at e0 (started in an earlier range): add its part.
  int64_t i = 0;
  if (e0 > 0) {
    const int64_t ic = last_row_at_or_before(a.row_ptr, a.n_dst, e0, lane);
    if (ic < a.n_dst && clamp_edge(a.row_ptr[ic], nnz) < e0) {
      const int64_t end = clamp_edge(a.row_ptr[ic + 1], nnz);
      accumulate<IdxT>(a, e0, e0, end < e1 ? end : e1, accp, ecol, eval, lane_edge,
                       lane_t, P);
      flush(a, ic, acc, P, lane, true);
      i = ic + 1;
    } else {
      // First row that starts at or after e0.
      i = last_row_at_or_before(a.row_ptr, a.n_dst, e0 - 1, lane) + 1;
    }
  }
  // Rows that start in [e0, e1) (the last wave also takes those starting at
  // nnz, i.e. trailing empty rows).
  for (; i < a.n_dst; ++i) {
    const int64_t start = clamp_edge(a.row_ptr[i], nnz);
    if (start >= e1 && !(last && start == nnz)) break;
    if (start < e0) continue;  // only with a row_ptr that decreases
    const int64_t end = clamp_edge(a.row_ptr[i + 1], nnz);
    const bool cut = end > e1;
    accumulate<IdxT>(a, e0, start, cut ? e1 : end, accp, ecol, eval, lane_edge,
                     lane_t, P);
    flush(a, i, acc, P, lane, cut);
  }
}

// ---------------------------------------------------------------------------
// Backward to the compressed features (SSpMM): grad_sp[j, t] = sum over the
// edges e = (i -> j) of val[e] * dY[i, sp_index[j, t]], i.e. A^T dY sampled
// at the survivors (review page: the backward reuses the forward's pattern
// with an outer-product dataflow and dense-row prefetching). The same CSR of
// A as the forward: wave w takes edges [w*C, (w+1)*C); for each row i with
// edges there it loads the dense row dY[i, :] into LDS once (coalesced),
// then every edge (i -> j) adds val * dY[i, sp_index[j, :]] into the k
// contiguous floats of grad_sp[j, :] with float atomics (grad_sp zeroed
// first). Lanes map to (edge slot, survivor) as in the forward.
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(kBlock) void zero_floats(float* p, int64_t count) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t q = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; q < count;
       q += stride)
    p[q] = 0.0f;
}

template <typename IdxT>
__global__ __launch_bounds__(kBlock) void sspmm_rows(SpgemmArgs a) {
  extern __shared__ float lds[];
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  const int wave_in_block =
      __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  // Per wave: the dense dY row (m_pad floats), then the staged edge range.
  float* dyrow = lds + static_cast<int64_t>(wave_in_block) * (a.m_pad + 2 * kEdgesPerWave);
  int* ecol = reinterpret_cast<int*>(dyrow + a.m_pad);
  float* eval = dyrow + a.m_pad + kEdgesPerWave;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * a.waves_per_block + wave_in_block;
  if (w >= a.waves || a.nnz == 0) return;
  const int64_t nnz = a.nnz;
  const int64_t e0 = w * a.chunk;
  const int64_t e1 = e0 + a.chunk < nnz ? e0 + a.chunk : nnz;
  for (int j = lane; j < kEdgesPerWave; j += kWave) {
    const int64_t e = e0 + j < e1 ? e0 + j : e1 - 1;
    // The CSR arrays are read once: non-temporal loads.
    ecol[j] = __builtin_nontemporal_load(a.col + e);
    eval[j] = __builtin_nontemporal_load(a.val + e);
  }
  __builtin_amdgcn_wave_barrier();
  const int k = a.k;
  const int P = a.slots;
  const int lane_edge = k <= kWave ? (lane < P * k ? lane / k : -1) : 0;
  const int lane_t = k <= kWave ? lane % k : lane;
  const int addr_edge = lane_edge < 0 ? 0 : lane_edge;
  const IdxT* sidx = static_cast<const IdxT*>(a.sp_index);
  const float* dy = a.sp_data;  // the backward's dense input, [n_dst, m]
  // Rows with edges in [e0, e1): from the row holding edge e0 on.
  for (int64_t i = last_row_at_or_before(a.row_ptr, a.n_dst, e0, lane); i < a.n_dst; ++i) {
    const int64_t rs = clamp_edge(a.row_ptr[i], nnz);
    if (rs >= e1) break;
    const int64_t re = clamp_edge(a.row_ptr[i + 1], nnz);
    const int64_t s0 = rs > e0 ? rs : e0;
    const int64_t s1 = re < e1 ? re : e1;
    if (s0 >= s1) continue;
    // Dense-row prefetch: dY[i, :] into LDS.
    for (int c = lane; c < a.m; c += kWave)
      dyrow[c] = __builtin_nontemporal_load(dy + i * a.m + c);  // read once
    __builtin_amdgcn_wave_barrier();
    constexpr int U = 8;  // steps whose index loads are issued together
    for (int64_t b0 = s0; b0 < s1; b0 += static_cast<int64_t>(U) * P) {
      for (int t0 = lane_t; t0 < k; t0 += kWave) {
        int c[U];
        float wv[U];
        int64_t dst[U];
        bool ok[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int64_t e = b0 + static_cast<int64_t>(u) * P + addr_edge;
          const int64_t ec = e < s1 ? e : s1 - 1;
          const int j = ecol[ec - e0];
          wv[u] = eval[ec - e0];
          const bool live = lane_edge >= 0 && e < s1 &&
                            static_cast<uint64_t>(static_cast<int64_t>(j)) <
                                static_cast<uint64_t>(a.n_src);
          const int64_t jj = live ? j : 0;
          c[u] = static_cast<int>(sidx[jj * k + t0]);
          dst[u] = jj * k + t0;
          ok[u] = live;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (ok[u] && static_cast<uint32_t>(c[u]) < static_cast<uint32_t>(a.m))
            unsafeAtomicAdd(a.y + dst[u], wv[u] * dyrow[c[u]]);  // hardware float atomic
        }
        if (k <= kWave) break;
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace spgemm_detail

// Both two-kernel launches below size and check every launch before the
// first one is enqueued, so that a configuration error enqueues nothing.
hipError_t launch_sspmm(SpgemmArgs a, bool u8_index, hipStream_t stream) {
  using namespace spgemm_detail;
  const int64_t count = a.n_src * a.k;
  a.chunk = kEdgesPerWave;
  a.waves = a.nnz > 0 ? (a.nnz + a.chunk - 1) / a.chunk : 0;
  a.m_pad = (a.m + 3) & ~3;
  a.slots = a.k <= kWave ? (kWave / a.k < 4 ? kWave / a.k : 4) : 1;
  const int per_wave_bytes =
      (a.m_pad + 2 * static_cast<int>(kEdgesPerWave)) * static_cast<int>(sizeof(float));
  int wpb = 65536 / per_wave_bytes;
  a.waves_per_block = wpb < 1 ? 1 : (wpb > kWavesPerBlock ? kWavesPerBlock : wpb);
  const int64_t blocks = (a.waves + a.waves_per_block - 1) / a.waves_per_block;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (count > 0) {
    int64_t zb = (count + kBlock - 1) / kBlock;
    zb = zb < 65536 ? zb : 65536;
    hipLaunchKernelGGL(zero_floats, dim3(static_cast<uint32_t>(zb)), dim3(kBlock), 0,
                       stream, a.y, count);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (a.nnz == 0) return hipSuccess;
  const size_t lds = static_cast<size_t>(a.waves_per_block) * per_wave_bytes;
  const dim3 block(kWave * a.waves_per_block);
  if (u8_index)
    hipLaunchKernelGGL(sspmm_rows<uint8_t>, dim3(static_cast<uint32_t>(blocks)), block, lds,
                       stream, a);
  else
    hipLaunchKernelGGL(sspmm_rows<int32_t>, dim3(static_cast<uint32_t>(blocks)), block, lds,
                       stream, a);
  return hipGetLastError();
}

hipError_t launch_spgemm(SpgemmArgs a, bool u8_index, hipStream_t stream) {
  using namespace spgemm_detail;
  a.chunk = kEdgesPerWave;
  a.waves = a.nnz > 0 ? (a.nnz + a.chunk - 1) / a.chunk : 1;
  a.m_pad = (a.m + 3) & ~3;
  a.slots = a.k <= kWave ? (kWave / a.k < 4 ? kWave / a.k : 4) : 1;
  const int per_wave_bytes =
      (a.slots * a.m_pad + 2 * static_cast<int>(kEdgesPerWave)) * static_cast<int>(sizeof(float));
  int wpb = 65536 / per_wave_bytes;
  a.waves_per_block = wpb < 1 ? 1 : (wpb > kWavesPerBlock ? kWavesPerBlock : wpb);
  const int64_t blocks = (a.waves + a.waves_per_block - 1) / a.waves_per_block;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  // Rows cut by a range boundary start at zero.
  if (a.waves > 1 && a.n_dst > 0) {
    const int64_t zb = (a.n_dst + kBlock - 1) / kBlock;
    if (zb > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(zero_cut_rows, dim3(static_cast<uint32_t>(zb)), dim3(kBlock), 0,
                       stream, a);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  const size_t lds = static_cast<size_t>(a.waves_per_block) * per_wave_bytes;
  const dim3 block(kWave * a.waves_per_block);
  if (u8_index)
    hipLaunchKernelGGL(spgemm_rows<uint8_t>, dim3(static_cast<uint32_t>(blocks)),
                       block, lds, stream, a);
  else
    hipLaunchKernelGGL(spgemm_rows<int32_t>, dim3(static_cast<uint32_t>(blocks)),
                       block, lds, stream, a);
  return hipGetLastError();
}

}  // namespace rtopk
