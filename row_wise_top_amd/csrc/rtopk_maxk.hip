// MaxK backward on gfx950: the gradient of each row's k survivors goes back
// to their columns of an otherwise zero dense row (MaxK-GNN review, "How
// MaxK-GNN works": only the survivors carry gradient, through the same
// sp_index the forward pass produced). The same scatter turns compressed
// rows (sp_data, sp_index) back into the dense MaxK output.
//
// Mapping. One wave64 assembles one row at a time in its own LDS area:
// 16-byte writes zero it, each lane writes its entries to their columns, and
// one coalesced pass stores the row. HBM sees every output byte written once,
// in whole lines, and nothing of the output is read. The grid is persistent;
// each wave loads the entries of its next row before it assembles the
// current one, with unconditional (clamped) loads so that the compiler's
// wait counts stay exact.
//
// Stores go through a buffer resource sized to the row: a store whose
// offset lies past the end is discarded by the hardware, so the tail of a
// row needs no branch.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rtopk_internal.h"

namespace rtopk {
namespace maxk_detail {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Columns one wave assembles per LDS pass in the general kernel, and the
// most the single-pass kernel handles.
constexpr int kChunk = 1024;
// Word 3 of a gfx9 buffer resource for untyped access (data format 32).
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t span(float* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(p, 0, bytes, kRsrcWord3);
}

// Zero the first 256*S columns of the wave's LDS row.
template <int S>
__device__ __forceinline__ void zero_row(u32x4* buf4, int lane) {
#pragma unroll
  for (int j = 0; j < S; ++j) buf4[j * kWave + lane] = u32x4{0u, 0u, 0u, 0u};
}

// Store columns [0, len) of the assembled row to dst. VEC: 16 bytes per lane
// (len and dst must be multiples of 4 floats / 16 bytes, so a 16-byte store
// lies wholly inside or wholly past the end); otherwise 4 bytes per lane.
template <int S, bool VEC>
__device__ __forceinline__ void store_row(const u32x4* buf4, float* dst,
                                          int len, int lane) {
  const __amdgpu_buffer_rsrc_t rs = span(dst, len * 4);
  if constexpr (VEC) {
#pragma unroll
    for (int j = 0; j < S; ++j) {
      __builtin_amdgcn_raw_buffer_store_b128(buf4[j * kWave + lane], rs,
                                             (j * 256 + 4 * lane) * 4, 0, 0);
    }
  } else {
    const uint32_t* buf = reinterpret_cast<const uint32_t*>(buf4);
#pragma unroll
    for (int j = 0; j < 4 * S; ++j) {
      __builtin_amdgcn_raw_buffer_store_b32(buf[j * kWave + lane], rs,
                                            (j * kWave + lane) * 4, 0, 0);
    }
  }
}

// Rows of length m <= 256*S with k <= 64*E entries, one LDS pass per row.
// Lane l holds entries l, 64 + l, ... of the row in registers.
template <typename IdxT, int S, int E, bool VEC>
__global__ __launch_bounds__(kBlock) void scatter_rows(ScatterArgs a) {
  __shared__ u32x4 lds[kWavesPerBlock][S * kWave];
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  const int wave_in_block =
      __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  u32x4* buf4 = lds[wave_in_block];
  uint32_t* buf = reinterpret_cast<uint32_t*>(buf4);
  const int64_t waves = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
  int64_t r = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave_in_block;
  if (r >= a.n) return;
  const int m = a.m, k = a.k;
  const IdxT* idx = static_cast<const IdxT*>(a.idx);
  // Entry e of this lane is entry 64e + lane of the row; lanes past k re-read
  // entry k - 1 (loads stay unconditional) and write nothing.
  int ent[E];
  bool live[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = e * kWave + lane;
    live[e] = i < k;
    ent[e] = i < k ? i : k - 1;
  }
  uint32_t g0[E], g1[E];
  int c0[E], c1[E];
  auto load = [&](int64_t row, uint32_t(&g)[E], int(&c)[E]) {
    const float* s = a.src + row * k;
    const IdxT* q = idx + row * k;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      g[e] = __float_as_uint(s[ent[e]]);
      c[e] = static_cast<int>(q[ent[e]]);
    }
  };
  load(r, g0, c0);
  for (;;) {
    // The next row of this wave (or, past the last one, this row again).
    load(r + waves < a.n ? r + waves : r, g1, c1);
    zero_row<S>(buf4, lane);
    // LDS operations of one wave complete in issue order; the barriers keep
    // the compiler from moving them across each other.
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int e = 0; e < E; ++e) {
      if (live[e] && static_cast<uint32_t>(c0[e]) < static_cast<uint32_t>(m))
        buf[c0[e]] = g0[e];
    }
    __builtin_amdgcn_wave_barrier();
    store_row<S, VEC>(buf4, a.out + r * m, m, lane);
    __builtin_amdgcn_wave_barrier();
    r += waves;
    if (r >= a.n) return;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      g0[e] = g1[e];
      c0[e] = c1[e];
    }
  }
}

// Any m <= kMaxRowLength and k <= m: the row in passes of kChunk columns,
// each pass reading all of the row's entries from memory.
template <typename IdxT, bool VEC>
__global__ __launch_bounds__(kBlock) void scatter_rows_chunked(ScatterArgs a) {
  constexpr int S = kChunk / 256;
  __shared__ u32x4 lds[kWavesPerBlock][S * kWave];
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  const int wave_in_block =
      __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  u32x4* buf4 = lds[wave_in_block];
  uint32_t* buf = reinterpret_cast<uint32_t*>(buf4);
  const int64_t waves = static_cast<int64_t>(gridDim.x) * kWavesPerBlock;
  const int m = a.m, k = a.k;
  const IdxT* idx = static_cast<const IdxT*>(a.idx);
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * kWavesPerBlock + wave_in_block;
       r < a.n; r += waves) {
    const float* s = a.src + r * k;
    const IdxT* q = idx + r * k;
    for (int c0 = 0; c0 < m; c0 += kChunk) {
      const int len = m - c0 < kChunk ? m - c0 : kChunk;
      zero_row<S>(buf4, lane);
      __builtin_amdgcn_wave_barrier();
      for (int i = lane; i < k; i += kWave) {
        const int col = static_cast<int>(q[i]) - c0;
        if (static_cast<uint32_t>(col) < static_cast<uint32_t>(len))
          buf[col] = __float_as_uint(s[i]);
      }
      __builtin_amdgcn_wave_barrier();
      store_row<S, VEC>(buf4, a.out + r * m + c0, len, lane);
      __builtin_amdgcn_wave_barrier();
    }
  }
}

using ScatterKernel = void (*)(ScatterArgs);

constexpr int bucket124(int v) { return v <= 1 ? 1 : (v <= 2 ? 2 : 4); }

template <typename IdxT, int S, int E>
ScatterKernel pick_vec(bool vec) {
  return vec ? scatter_rows<IdxT, S, E, true> : scatter_rows<IdxT, S, E, false>;
}

template <typename IdxT, int S>
ScatterKernel pick_e(int e, bool vec) {
  switch (e) {
    case 1: return pick_vec<IdxT, S, 1>(vec);
    case 2: return pick_vec<IdxT, S, 2>(vec);
    default: return pick_vec<IdxT, S, 4>(vec);
  }
}

template <typename IdxT>
ScatterKernel pick(int m, int k, bool vec) {
  if (m <= kChunk && k <= 4 * kWave) {
    const int s = bucket124((m + 255) / 256);
    const int e = bucket124((k + kWave - 1) / kWave);
    switch (s) {
      case 1: return pick_e<IdxT, 1>(e, vec);
      case 2: return pick_e<IdxT, 2>(e, vec);
      default: return pick_e<IdxT, 4>(e, vec);
    }
  }
  return vec ? scatter_rows_chunked<IdxT, true> : scatter_rows_chunked<IdxT, false>;
}

}  // namespace maxk_detail

hipError_t launch_scatter(const ScatterArgs& a, bool u8_index,
                          hipStream_t stream) {
  using namespace maxk_detail;
  const bool vec =
      a.m % 4 == 0 && (reinterpret_cast<uintptr_t>(a.out) & 15u) == 0;
  const ScatterKernel fn =
      u8_index ? pick<uint8_t>(a.m, a.k, vec) : pick<int32_t>(a.m, a.k, vec);
  int device = 0;
  hipError_t err = hipGetDevice(&device);
  if (err != hipSuccess) return err;
  const int64_t blocks_needed = (a.n + kWavesPerBlock - 1) / kWavesPerBlock;
  const int64_t resident =
      static_cast<int64_t>(cu_count(device)) *
      resident_blocks(reinterpret_cast<const void*>(fn), device);
  const int64_t grid = blocks_needed < resident ? blocks_needed : resident;
  hipLaunchKernelGGL(fn, dim3(static_cast<uint32_t>(grid)), dim3(kBlock), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace rtopk
