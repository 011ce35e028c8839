// MaxK backward on gfx950: the gradient of each row's k survivors goes back
// to their columns of an otherwise zero dense row (MaxK-GNN review, "How
// MaxK-GNN works": only the survivors carry gradient, through the same
// sp_index the forward pass produced). The same scatter turns compressed
// rows (sp_data, sp_index) back into the dense MaxK output.
//
// Mapping. A wave64 assembles a batch of consecutive rows in its own LDS
// area: 16-byte writes zero it, each lane writes its entries to their
// columns, and one coalesced pass stores the rows. HBM sees every output
// byte written once, in whole lines, and nothing of the output is read.
// Rows up to 1024 long take one batch per wave (see scatter_rows); longer
// rows, or more than 256 entries per row, go through a persistent kernel
// that assembles each row in passes of 1024 columns.
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
// Cache policy of the dense-row stores (gfx950 encoding, bit 1 =
// non-temporal): the rows are written once, in whole lines. The entry loads
// keep the default policy (measured at 262,144 x 256, k = 32: 53.9 us with
// non-temporal stores only, 55.4 us with non-temporal loads too, 56.5 us
// with neither).
constexpr int kNT = 2;

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
                                             (j * 256 + 4 * lane) * 4, 0, kNT);
    }
  } else {
    const uint32_t* buf = reinterpret_cast<const uint32_t*>(buf4);
#pragma unroll
    for (int j = 0; j < 4 * S; ++j) {
      __builtin_amdgcn_raw_buffer_store_b32(buf[j * kWave + lane], rs,
                                            (j * kWave + lane) * 4, 0, kNT);
    }
  }
}

// LDS floats each wave assembles rows in (4 KB): 32 resident waves per CU
// then use 128 KB of the 160 KB.
constexpr int kBatchFloats = 1024;

// Waves per block of the scatter kernels.
constexpr int kScatterWaves = 4;
constexpr int kScatterBlock = kWave * kScatterWaves;

// Rows of length m <= 256*S, in batches of B consecutive rows,
// B = min(kBatchFloats / (256*S), 64*EB / k) >= 1 (host checked). One wave
// takes one batch and exits: it loads the batch's B*k entries (contiguous in
// memory; lane l holds entries t = 64e + l, which belong to row t / k of the
// batch), assembles the B rows in LDS and stores them, B*m contiguous floats.
//
// Why one batch per wave rather than a persistent loop: on this GPU loads
// and stores complete in issue order on one counter, so in a loop the wait
// for the next entries also waits for the stores issued before them, and
// each wave ends up with little output in flight. A wave that loads first
// and stores last never waits for a store; the hardware keeps the grid's
// waves streaming (measured at the 262,144 x 256 shape: 63.8 us for the
// persistent loop, about 20% less one-shot).
template <typename IdxT, int S, int EB, bool VEC>
__global__ __launch_bounds__(kScatterBlock) void scatter_rows(ScatterArgs a, int B) {
  constexpr int kPad = 256 * S;                     // LDS row stride (floats)
  constexpr int kMaxB = kBatchFloats / kPad;        // rows the LDS area holds
  __shared__ u32x4 lds[kScatterWaves][kBatchFloats / 4];
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  const int wave_in_block =
      __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  u32x4* buf4 = lds[wave_in_block];
  uint32_t* buf = reinterpret_cast<uint32_t*>(buf4);
  const int64_t j = static_cast<int64_t>(blockIdx.x) * kScatterWaves + wave_in_block;
  const int64_t row0 = j * B;
  if (row0 >= a.n) return;
  const int m = a.m, k = a.k;
  // The batch's entries through buffer resources that end at the arrays'
  // end: lanes past it read 0 (their row lies past n and writes nothing).
  const int64_t base = row0 * k;
  const int64_t rest = a.n * k - base;
  // Capped so that the byte count stays an int (a batch reads at most 256).
  const int count = rest < 0x1fffffff ? static_cast<int>(rest) : 0x1fffffff;
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.src + base), 0, count * 4, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t ri = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<IdxT*>(static_cast<const IdxT*>(a.idx) + base), 0,
      count * static_cast<int>(sizeof(IdxT)), kRsrcWord3);
  uint32_t g[EB];
  int c[EB], brow[EB];
#pragma unroll
  for (int e = 0; e < EB; ++e) {
    const int t = e * kWave + lane;
    g[e] = __builtin_amdgcn_raw_buffer_load_b32(rv, t * 4, 0, 0);
    if constexpr (sizeof(IdxT) == 1)
      c[e] = __builtin_amdgcn_raw_buffer_load_b8(ri, t, 0, 0);
    else
      c[e] = static_cast<int>(__builtin_amdgcn_raw_buffer_load_b32(ri, t * 4, 0, 0));
    brow[e] = t < B * k ? t / k : -1;
  }
#pragma unroll
  for (int i = 0; i < kBatchFloats / 256; ++i)
    buf4[i * kWave + lane] = u32x4{0u, 0u, 0u, 0u};
  // LDS operations of one wave complete in issue order; the barriers keep
  // the compiler from moving them across each other.
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int e = 0; e < EB; ++e) {
    const bool ok = brow[e] >= 0 && row0 + brow[e] < a.n &&
                    static_cast<uint32_t>(c[e]) < static_cast<uint32_t>(m);
    if (ok) buf[brow[e] * kPad + c[e]] = g[e];
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int b = 0; b < kMaxB; ++b) {
    const bool real = b < B && row0 + b < a.n;
    const __amdgpu_buffer_rsrc_t rs = span(a.out + (row0 + b) * m, real ? m * 4 : 0);
    if constexpr (VEC) {
#pragma unroll
      for (int i = 0; i < S; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(buf4[(b * kPad) / 4 + i * kWave + lane],
                                               rs, (i * 256 + 4 * lane) * 4, 0, kNT);
    } else {
#pragma unroll
      for (int i = 0; i < 4 * S; ++i)
        __builtin_amdgcn_raw_buffer_store_b32(buf[b * kPad + i * kWave + lane], rs,
                                              (i * kWave + lane) * 4, 0, kNT);
    }
  }
}

// Any m <= kMaxRowLength and k <= m: the row in passes of kChunk columns,
// each pass reading all of the row's entries from memory.
template <typename IdxT, bool VEC>
__device__ __forceinline__ void scatter_rows_chunked_body(const ScatterArgs& a) {
  constexpr int S = kChunk / 256;
  __shared__ u32x4 lds[kScatterWaves][S * kWave];
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  const int wave_in_block =
      __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  u32x4* buf4 = lds[wave_in_block];
  uint32_t* buf = reinterpret_cast<uint32_t*>(buf4);
  const int64_t waves = static_cast<int64_t>(gridDim.x) * kScatterWaves;
  const int m = a.m, k = a.k;
  const IdxT* idx = static_cast<const IdxT*>(a.idx);
  for (int64_t r = static_cast<int64_t>(blockIdx.x) * kScatterWaves + wave_in_block;
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

using ScatterKernel = void (*)(ScatterArgs, int);

constexpr int bucket124(int v) { return v <= 1 ? 1 : (v <= 2 ? 2 : 4); }

template <typename IdxT, bool VEC>
__global__ __launch_bounds__(kScatterBlock) void scatter_rows_chunked_entry(ScatterArgs a, int) {
  scatter_rows_chunked_body<IdxT, VEC>(a);
}

template <typename IdxT, int S, int EB>
ScatterKernel pick_vec(bool vec) {
  return vec ? scatter_rows<IdxT, S, EB, true> : scatter_rows<IdxT, S, EB, false>;
}

template <typename IdxT, int S>
ScatterKernel pick_e(int eb, bool vec) {
  switch (eb) {
    case 1: return pick_vec<IdxT, S, 1>(vec);
    case 2: return pick_vec<IdxT, S, 2>(vec);
    default: return pick_vec<IdxT, S, 4>(vec);
  }
}

// The kernel for (m, k), the rows per batch it takes (1 for the chunked
// kernel, which ignores it) and whether it is the chunked (persistent) one.
template <typename IdxT>
ScatterKernel pick(int m, int k, bool vec, int* rows_per_batch, bool* chunked) {
  if (m <= kChunk && k <= 4 * kWave) {
    const int s = bucket124((m + 255) / 256);
    const int max_b = kBatchFloats / (256 * s);
    // Entries per lane: enough for max_b rows, at most 4 (256 per batch).
    const int eb = bucket124((max_b * k + kWave - 1) / kWave);
    int b = (kWave * eb) / k;
    b = b < max_b ? b : max_b;
    *rows_per_batch = b < 1 ? 1 : b;
    *chunked = false;
    switch (s) {
      case 1: return pick_e<IdxT, 1>(eb, vec);
      case 2: return pick_e<IdxT, 2>(eb, vec);
      default: return pick_e<IdxT, 4>(eb, vec);
    }
  }
  *rows_per_batch = 1;
  *chunked = true;
  return vec ? scatter_rows_chunked_entry<IdxT, true>
             : scatter_rows_chunked_entry<IdxT, false>;
}

}  // namespace maxk_detail

hipError_t launch_scatter(const ScatterArgs& a, bool u8_index,
                          hipStream_t stream) {
  using namespace maxk_detail;
  const bool vec =
      a.m % 4 == 0 && (reinterpret_cast<uintptr_t>(a.out) & 15u) == 0;
  int rows_per_batch = 1;
  bool chunked = false;
  const ScatterKernel fn =
      u8_index ? pick<uint8_t>(a.m, a.k, vec, &rows_per_batch, &chunked)
               : pick<int32_t>(a.m, a.k, vec, &rows_per_batch, &chunked);
  int device = 0;
  hipError_t err = hipGetDevice(&device);
  if (err != hipSuccess) return err;
  const int64_t batches = (a.n + rows_per_batch - 1) / rows_per_batch;
  const int64_t blocks_needed = (batches + kScatterWaves - 1) / kScatterWaves;
  int64_t grid = blocks_needed;
  if (chunked) {
    // The chunked kernel loops over rows: a persistent grid.
    const int64_t resident =
        static_cast<int64_t>(cu_count(device)) *
        resident_blocks(reinterpret_cast<const void*>(fn), kScatterBlock, device);
    grid = blocks_needed < resident ? blocks_needed : resident;
  }
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fn, dim3(static_cast<uint32_t>(grid)), dim3(kScatterBlock), 0,
                     stream, a, rows_per_batch);
  return hipGetLastError();
}

}  // namespace rtopk
