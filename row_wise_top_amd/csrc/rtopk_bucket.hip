// Bucketed top-k with short buckets on gfx950 ("Approximate Top-k for
// Increased Parallelism", abstract: many small independent top-k selections
// in place of one). Each input row is split into b contiguous buckets of
// w = m / b columns and each bucket keeps its kb = k / b largest elements
// (ties to the lowest column), listed in column order.
//
// When buckets are short (w <= 64) a wave-wide search per bucket would leave
// most lanes idle and pay the search's fixed cost b times per row. Here one
// lane owns one bucket instead: it loads the bucket's w elements and finds
// its kb best in registers. Up to two survivors: sorted insertion of
// (value, column) pairs, strictly greater values moving up so that among
// equal values the earlier column stays ahead. More: the kb largest values
// by median-of-three insertion, then one pass in column order that keeps
// every element above the kb-th largest value and the first few equal to
// it. A wave takes 64 consecutive buckets, so its loads and stores cover
// one contiguous stretch of the input and of the outputs. Buckets of 65 to
// 128 columns keeping at most 16 take four lanes each (bucket_quads below).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rtopk_internal.h"

namespace rtopk {
namespace bucket_detail {

// Word 3 of a gfx9 buffer resource for untyped access (data format 32).
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy of the bucket loads: the default one. The input is read once,
// but the lanes of a wave share lines between their loads, and the kernel
// reads survivors back from the bucket; non-temporal loads (gfx950 policy
// bit 1) measured 109 -> 190 us at 262,144 x 256 with 8 buckets.
constexpr int kLoadPolicy = 0;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// acc = 2 * acc + (x < t), from the sign of x - t: for finite x and t the
// difference is rounded once, so it is negative exactly when x < t, except
// that -0 - (+0) is -0. Callers pass a zero threshold as -0 (see
// zero_as_minus), and x - (-0) is +0 for x = +-0. One subtraction and one
// funnel shift per place, with no lane mask.
__device__ __forceinline__ uint32_t shift_in_lt(uint32_t acc, float x, float t) {
  return (acc << 1) | (__float_as_uint(x - t) >> 31);
}
__device__ __forceinline__ float zero_as_minus(float t) {
  return __uint_as_float(t == 0.0f ? 0x80000000u : __float_as_uint(t));
}
// acc = 2 * acc + (x == t): the compare's lane mask is the carry-in of one
// add (two instructions, no mask logic).
__device__ __forceinline__ void shift_in_eq(uint32_t& acc, float x, float t) {
  asm("v_cmp_eq_f32 vcc, %2, %1\n\tv_addc_co_u32 %0, vcc, %0, %0, vcc"
      : "+v"(acc)
      : "v"(x), "v"(t)
      : "vcc");
}

// One lane per bucket row g (a.n of them): w = a.m <= W columns, kb = a.k
// <= KB survivors, a.buckets buckets per input row. The bucket's elements
// are x[g*w, g*w + w) and its survivors go to entries [g*kb, g*kb + kb) of
// the outputs, with columns relative to the input row ((g mod b) * w + j).
// VEC: w is a multiple of 4 and x 16-byte aligned, so the bucket is read
// with 16-byte loads.
//
// The buffer resources start at the wave's first bucket (they must be the
// same for every lane) and end at the wave's last one or the end of the
// arrays: lanes past the end read zeros and their stores are dropped.
//
// Buckets of more than 16 columns (W >= 32) with 16-byte loads go through
// LDS: a lane's 16-byte loads at a 128-byte stride would make every load
// instruction touch 64 lines (measured: a load-only version of the kernel
// ran at 95 us for 262,144 x 256 in 8 buckets, against 54 us with 16
// columns). The wave instead reads its buckets into LDS with each load
// instruction covering 1 KB of consecutive buckets (256 / W of them), and
// each lane takes its bucket from there. (Staging a 64-column bucket in two
// rounds of 32, at 9 KB of LDS per wave instead of 17 KB and twice the
// occupancy, measured slower: 167 against 108 us, the survivors then being
// read back from memory rather than LDS.)
template <int W, bool VEC>
constexpr bool lane_stage() {
  return VEC && W >= 32;
}

// One lane's bucket of a group of 64 consecutive buckets starting at bucket
// g0 (live of them exist): v holds its W places (-inf past w), `row` is its
// LDS row when the group was staged (values of survivors are read back from
// there), else the bucket is read again from memory through rx at byte
// offset `base`. Finds the bucket's kb best and writes them lowest column
// first to entries [g*kb, g*kb + kb) of the outputs.
template <int W, int KB, bool kStage, typename IdxT>
__device__ __forceinline__ void select_bucket(const SelectArgs& a, int64_t g0, int live, int lane,
                                              const float (&v)[W], const float* row,
                                              __amdgpu_buffer_rsrc_t rx, int base) {
  const int w = a.m, kb = a.k;
  // Column of the bucket's first element within the input row.
  const uint32_t b = static_cast<uint32_t>(a.buckets);
  const uint32_t r0 = g0 < 0x100000000LL ? static_cast<uint32_t>(g0) % b
                                         : static_cast<uint32_t>(g0 % a.buckets);
  const uint32_t first = ((r0 + static_cast<uint32_t>(lane)) % b) * static_cast<uint32_t>(w);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      a.out_val + g0 * kb, 0, live * kb * 4, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t ri = __builtin_amdgcn_make_buffer_rsrc(
      static_cast<IdxT*>(a.out_idx) + g0 * kb, 0,
      live * kb * static_cast<int>(sizeof(IdxT)), kRsrcWord3);
  // Entry i of the lane's output; places past kb store past the resources'
  // end, where the hardware drops them.
  auto put = [&](int i, float x, uint32_t col) {
    const int e = i < kb ? lane * kb + i : (1 << 28);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), rv, e * 4, 0, 0);
    if constexpr (sizeof(IdxT) == 1)
      __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(first + col), ri, e, 0, 0);
    else
      __builtin_amdgcn_raw_buffer_store_b32(first + col, ri, e * 4, 0, 0);
  };
  // All KB entries of the lane, when kb == KB and both outputs are 16-byte
  // aligned: the lane's entries are then one contiguous piece of each
  // output, stored with the widest stores (one 16-byte value store per four
  // entries), so each store instruction writes whole lines. Entry by entry,
  // every store instruction wrote 64 scattered words. Lanes past the
  // group's end store past the resources' end (dropped).
  const bool vec_out = kb == KB && ((reinterpret_cast<uintptr_t>(a.out_val) |
                                     reinterpret_cast<uintptr_t>(a.out_idx)) & 15) == 0;
  auto put_all = [&](const uint32_t (&xb)[KB], const int (&col)[KB]) {
    if (KB > 1 && vec_out) {
      if constexpr (KB == 2) {
        const u32x2 xv = {xb[0], xb[1]};
        __builtin_amdgcn_raw_buffer_store_b64(xv, rv, lane * 8, 0, 0);
        if constexpr (sizeof(IdxT) == 1) {
          const uint32_t iv = ((first + col[0]) & 0xffu) | (((first + col[1]) & 0xffu) << 8);
          __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(iv), ri, lane * 2, 0, 0);
        } else {
          const u32x2 iv = {first + col[0], first + col[1]};
          __builtin_amdgcn_raw_buffer_store_b64(iv, ri, lane * 8, 0, 0);
        }
      } else if constexpr (KB >= 4) {
#pragma unroll
        for (int c = 0; c < KB; c += 4) {
          const u32x4 xv = {xb[c], xb[c + 1], xb[c + 2], xb[c + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(xv, rv, (lane * KB + c) * 4, 0, 0);
          if constexpr (sizeof(IdxT) == 1) {
            uint32_t iv = 0;
#pragma unroll
            for (int j = 3; j >= 0; --j) iv = (iv << 8) | ((first + col[c + j]) & 0xffu);
            __builtin_amdgcn_raw_buffer_store_b32(iv, ri, lane * KB + c, 0, 0);
          } else {
            const u32x4 iv = {first + col[c], first + col[c + 1], first + col[c + 2],
                              first + col[c + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(iv, ri, (lane * KB + c) * 4, 0, 0);
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < KB; ++i) put(i, __uint_as_float(xb[i]), static_cast<uint32_t>(col[i]));
    }
  };
  if constexpr (KB <= 2) {
    // The KB best so far with their columns, largest first. Empty places
    // hold -inf (inputs are finite, so the first KB elements always enter).
    // The survivors are carried as bits (integer selects): a float select
    // `x > t ? x : t` may be folded into a maximum, which need not keep the
    // sign of a zero that ties.
    uint32_t tb[KB];
    int tc[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      tb[i] = __float_as_uint(-__builtin_inff());
      tc[i] = i;
    }
#pragma unroll
    for (int j = 0; j < W; ++j) {
      // Straight-line code over all W places (no loop the compiler could
      // roll up and index registers in).
      const float x = v[j];
      const uint32_t xb = __float_as_uint(x);
      bool gt[KB];
#pragma unroll
      for (int i = 0; i < KB; ++i) gt[i] = x > __uint_as_float(tb[i]);
      // Insert x above every element it beats: place i takes the element of
      // place i - 1 if x beats that one too, else x if x beats place i.
#pragma unroll
      for (int i = KB - 1; i > 0; --i) {
        tb[i] = gt[i - 1] ? tb[i - 1] : (gt[i] ? xb : tb[i]);
        tc[i] = gt[i - 1] ? tc[i - 1] : (gt[i] ? j : tc[i]);
      }
      tb[0] = gt[0] ? xb : tb[0];
      tc[0] = gt[0] ? j : tc[0];
    }
    if constexpr (KB == 2) {
      // Column order (with kb == 1 the second place is dropped anyway).
      const bool sw = kb == 2 && tc[0] > tc[1];
      const uint32_t b0 = tb[0];
      const int c0 = tc[0];
      tb[0] = sw ? tb[1] : tb[0];
      tc[0] = sw ? tc[1] : tc[0];
      tb[1] = sw ? b0 : tb[1];
      tc[1] = sw ? c0 : tc[1];
    }
    put_all(tb, tc);
  } else {
    // The KB largest values (a multiset, largest first) by median-of-three
    // insertion: with tv sorted, place i becomes med3(tv[i-1], x, tv[i]).
    float tv[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) tv[i] = -__builtin_inff();
#pragma unroll
    for (int j = 0; j < W; ++j) {
      const float x = v[j];
#pragma unroll
      for (int i = KB - 1; i > 0; --i) tv[i] = __builtin_amdgcn_fmed3f(tv[i - 1], x, tv[i]);
      tv[0] = fmaxf(tv[0], x);
    }
    // The kb-th largest value and how many of the kb largest equal it.
    float thr = tv[0];
#pragma unroll
    for (int i = 1; i < KB; ++i) thr = i < kb ? tv[i] : thr;
    int need_eq = 0;
#pragma unroll
    for (int i = 0; i < KB; ++i) need_eq += (i < kb && tv[i] == thr) ? 1 : 0;
    // Bit masks of the places at or above thr: place j at bit 31 - (j mod
    // 32) of word j / 32 (built from the places below thr). Without surplus
    // ties these are the survivors.
    constexpr int NW = (W + 31) / 32;
    uint32_t keep[NW];
    int count = 0;
    const float thr_s = zero_as_minus(thr);
#pragma unroll
    for (int q = 0; q < NW; ++q) {
      constexpr int kLast = W < 32 ? W : 32;  // places per word
      uint32_t below = 0;
#pragma unroll
      for (int j = 0; j < kLast; ++j) below = shift_in_lt(below, v[32 * q + j], thr_s);
      keep[q] = ~below << (32 - kLast);
      count += __builtin_popcount(keep[q]);
    }
    if (__builtin_amdgcn_ballot_w64(count > kb) != 0) {
      // Some lane has more elements equal to thr than the need_eq the kb
      // largest hold: keep every place above thr and the need_eq lowest
      // places (first words, highest bits) equal to it.
      uint32_t equal[NW];
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        constexpr int kLast = W < 32 ? W : 32;
        equal[q] = 0;
#pragma unroll
        for (int j = 0; j < kLast; ++j) shift_in_eq(equal[q], v[32 * q + j], thr);
        equal[q] <<= 32 - kLast;
        keep[q] &= ~equal[q];
      }
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        bool done = i >= need_eq;
#pragma unroll
        for (int q = 0; q < NW; ++q) {
          const uint32_t top = equal[q] != 0u ? 0x80000000u >> __builtin_clz(equal[q]) : 0u;
          const bool take = !done && top != 0u;
          keep[q] |= take ? top : 0u;
          equal[q] ^= take ? top : 0u;
          done = done || take;
        }
      }
    }
    // Emit them lowest column first: the columns, then the values (read
    // again from the bucket, from LDS or from its line in the cache, which
    // keeps the original bits; the reads are issued together), then the
    // stores, as straight-line code (a branch between survivors made each
    // read wait by itself).
    int cols[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      int col = 0;
      bool found = false;
#pragma unroll
      for (int q = 0; q < NW; ++q) {
        const bool here = !found && keep[q] != 0u;
        const int c = keep[q] != 0u ? __builtin_clz(keep[q]) : 0;
        col = here ? 32 * q + c : col;
        keep[q] &= here ? ~(0x80000000u >> c) : ~0u;
        found = found || here;
      }
      cols[i] = col;
    }
    uint32_t xs[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      if constexpr (kStage)
        xs[i] = __float_as_uint(row[cols[i]]);
      else
        xs[i] = __builtin_amdgcn_raw_buffer_load_b32(rx, base + cols[i] * 4, 0, 0);
    }
    put_all(xs, cols);
  }
}

// Waves per block: one, so that a block's LDS (17 KB for the 64-column
// stage) frees as soon as its wave ends (measured 1-2% faster than four
// waves for 8 and 32 buckets of 256 columns, 7% for 4 buckets).
constexpr int kLaneWaves = 1;
constexpr int kSimdsPerCu = 4;
constexpr int kMaxStagedWavesPerCu = 3 * kSimdsPerCu;

// Staged groups: each wave takes groups blockIdx.x, blockIdx.x + gridDim.x,
// ... (the host sizes the grid to what is resident, never more than the
// groups there are). The loads of a wave's next group are issued into
// registers before the current group's selection, so every wave keeps a
// group's loads in flight while it works; with one group per wave the
// loads of a wave waited behind its own selection and the 9 waves per CU
// that the LDS allows left the memory system idle part of the time.
template <int W>
__device__ __forceinline__ void load_group(const SelectArgs& a, int64_t g0, int live, int lane,
                                           u32x4 (&q)[W / 4]) {
  const int w = a.m;
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(a.x + g0 * w), 0, live * w * 4, kRsrcWord3);
  // Chunk c = 64 i + lane (16 bytes) is place 4 (c mod (W/4)) of bucket
  // c / (W/4); chunks past the group's buckets read zeros and are not
  // written to LDS below.
  constexpr int kChunks = W / 4;  // chunks per bucket
#pragma unroll
  for (int i = 0; i < W / 4; ++i) {
    const int c = i * kWave + lane;
    const int bkt = c / kChunks;
    const int p = 4 * (c % kChunks);
    q[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, (bkt * w + p) * 4, 0, kLoadPolicy);
  }
}

template <int W, int KB, bool VEC, typename IdxT>
__global__ __launch_bounds__(kLaneWaves * kWave) void bucket_lanes(SelectArgs a) {
  constexpr bool kStage = lane_stage<W, VEC>();
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  const int w = a.m;
  if constexpr (kStage) {
    // LDS row of a lane: W + 4 floats (16-byte aligned; the skew of 4 banks
    // per row keeps 8 consecutive lanes on distinct banks for both the
    // writes and the reads below).
    constexpr int kStride = W + 4;
    constexpr int kChunks = W / 4;
    __shared__ u32x4 stage[kWave * kStride / 4];
    const int64_t groups = (a.n + kWave - 1) / kWave;
    int64_t grp = blockIdx.x;
    if (grp >= groups) return;
    auto live_of = [&](int64_t g) {
      const int64_t rest = a.n - g * kWave;
      return rest < kWave ? static_cast<int>(rest) : kWave;
    };
    u32x4 q[W / 4];
    load_group<W>(a, grp * kWave, live_of(grp), lane, q);
    // Places past w of every LDS row hold -inf for the whole kernel (the
    // staging below writes places < w only), which takes them out of every
    // comparison (the inputs are finite). Written after the first loads
    // are issued, so that they do not wait behind it.
    if (w < W) {
      constexpr u32x4 kNegInf = {0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u};
      for (int i = lane; i < kWave * kStride / 4; i += kWave) stage[i] = kNegInf;
    }
    for (;;) {
      const int64_t g0 = grp * kWave;
      const int live = live_of(grp);
#pragma unroll
      for (int i = 0; i < W / 4; ++i) {
        const int c = i * kWave + lane;
        const int bkt = c / kChunks;
        const int p = 4 * (c % kChunks);
        if (p < w && bkt < live) stage[(bkt * kStride + p) / 4] = q[i];
      }
      // LDS operations of one wave complete in issue order; the barriers
      // keep the compiler from moving the reads above the writes (and, at
      // the loop's end, the next group's writes above this group's reads).
      __builtin_amdgcn_wave_barrier();
      asm volatile("" ::: "memory");
      const int64_t next = grp + gridDim.x;
      if (next < groups) load_group<W>(a, next * kWave, live_of(next), lane, q);
      float v[W];
#pragma unroll
      for (int j = 0; j < W; j += 4) {
        const u32x4 e = stage[(lane * kStride + j) / 4];
        v[j] = __uint_as_float(e.x);
        v[j + 1] = __uint_as_float(e.y);
        v[j + 2] = __uint_as_float(e.z);
        v[j + 3] = __uint_as_float(e.w);
      }
      const __amdgpu_buffer_rsrc_t none = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(a.x), 0, 0, kRsrcWord3);
      select_bucket<W, KB, true, IdxT>(a, g0, live, lane, v,
                                       reinterpret_cast<const float*>(stage) + lane * kStride,
                                       none, 0);
      if (next >= groups) break;
      grp = next;
      __builtin_amdgcn_wave_barrier();
      asm volatile("" ::: "memory");
    }
  } else {
    const int64_t g0 = static_cast<int64_t>(blockIdx.x) * kWave;
    if (g0 >= a.n) return;
    const int live = a.n - g0 < kWave ? static_cast<int>(a.n - g0) : kWave;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(a.x + g0 * w), 0, live * w * 4, kRsrcWord3);
    // Elements past the bucket (j >= w) belong to the next one and are
    // never considered.
    const int base = lane * w * 4;
    float v[W];
    if constexpr (VEC) {
#pragma unroll
      for (int j = 0; j < W; j += 4) {
        const u32x4 q = __builtin_amdgcn_raw_buffer_load_b128(rx, base + j * 4, 0, kLoadPolicy);
        v[j] = __uint_as_float(q.x);
        v[j + 1] = __uint_as_float(q.y);
        v[j + 2] = __uint_as_float(q.z);
        v[j + 3] = __uint_as_float(q.w);
      }
    } else {
#pragma unroll
      for (int j = 0; j < W; ++j)
        v[j] = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(rx, base + j * 4, 0, kLoadPolicy));
    }
    if (w < W) {
#pragma unroll
      for (int j = 0; j < W; ++j) v[j] = j < w ? v[j] : -__builtin_inff();
    }
    select_bucket<W, KB, false, IdxT>(a, g0, live, lane, v, nullptr, rx, base);
  }
}

// Batcher's odd-even merge sort network on N places, as a table of
// compare-exchange pairs (a < b), built at compile time so that the
// unrolled loops below index registers with constants only.
template <int N>
struct OddEvenMergeNet {
  int count = 0;
  int a[N * N] = {};
  int b[N * N] = {};
  constexpr OddEvenMergeNet() {
    for (int p = 1; p < N; p <<= 1)
      for (int k = p; k >= 1; k >>= 1)
        for (int j = k % p; j + k < N; j += 2 * k)
          for (int i = 0; i < k && i + j + k < N; ++i)
            if ((i + j) / (2 * p) == (i + j + k) / (2 * p)) {
              a[count] = i + j;
              b[count] = i + j + k;
              ++count;
            }
  }
};

// Sorts v into descending order.
template <int N>
__device__ __forceinline__ void sort_desc(float (&v)[N]) {
  constexpr OddEvenMergeNet<N> net{};
#pragma unroll
  for (int c = 0; c < net.count; ++c) {
    const float x = v[net.a[c]], y = v[net.b[c]];
    v[net.a[c]] = fmaxf(x, y);
    v[net.b[c]] = fminf(x, y);
  }
}

// t (descending) becomes the N largest of t and u (both descending): the
// elementwise maximum of t and u reversed holds them as a bitonic sequence,
// which half-cleaners at distances N/2 .. 1 sort.
template <int N>
__device__ __forceinline__ void merge_top_desc(float (&t)[N], const float (&u)[N]) {
#pragma unroll
  for (int i = 0; i < N; ++i) t[i] = fmaxf(t[i], u[N - 1 - i]);
#pragma unroll
  for (int d = N / 2; d >= 1; d /= 2) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if ((i & d) == 0) {
        const float hi = fmaxf(t[i], t[i + d]);
        const float lo = fminf(t[i], t[i + d]);
        t[i] = hi;
        t[i + d] = lo;
      }
    }
  }
}

// Buckets of 65 to 128 columns keeping at most 16 (w a multiple of 4, x
// 16-byte aligned): four lanes per bucket, lane l taking bucket l mod 16 of
// a group of 16 and its quarter h = l / 16 (columns [32h, 32h + 32)). Each
// lane finds the KB largest values of its quarter (median-of-three
// insertion, or two sorted batches of 16 merged); the sorted lists of lanes
// l and l ^ 16 (the other quarter of the same half), then those of the two
// halves, are exchanged with lane swaps and merged (merge_top_desc), so all
// four lanes hold the bucket's KB largest values. Each lane then keeps its
// places at or above the kb-th of them; surplus ties at that value are
// dropped from the highest columns (lower quarters keep their equal places
// first). Each quarter emits its survivors after those of the quarters
// before it, so the bucket's entries are in column order. Persistent grid and staging as in bucket_lanes: the
// next group's loads are in flight while the current group is selected.
//
// The layout is set by occupancy. With two lanes per bucket (32 buckets, a
// 17 KB stage and 64 places per lane) the kernel held 235 registers and ran
// two waves per SIMD, its vector unit idle half the time (waiting on LDS
// and permutes); four lanes per bucket halve the stage (16 buckets, 8.4 KB)
// and the registers (three waves per SIMD, as many as the host launches),
// at the cost of a second cross-lane merge.

// A value of lane l and of its partner l ^ D (D = 16 or 32), through the
// gfx950 lane swaps: lo receives the value of the lane whose bit D is clear,
// hi that of the lane whose bit D is set (each lane gets both; swapping x
// with itself exchanges the two rows, or halves, of the wave).
template <int D>
__device__ __forceinline__ void swap_rows(uint32_t x, uint32_t& lo, uint32_t& hi) {
  static_assert(D == 16 || D == 32, "row or half swaps");
  if constexpr (D == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    lo = r[0];
    hi = r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    lo = r[0];
    hi = r[1];
  }
}

constexpr int kQuadWidth = kQuadBucketWidth;   // bucket capacity
constexpr int kQuadGroup = kWave / 4;          // buckets per group
constexpr int kQuarter = kQuadWidth / 4;       // places per lane

// VEC_OUT: both outputs are 16-byte aligned (the outputs are then stored
// in 16-byte pieces; every group's stretch starts at a multiple of 16 kb
// entries).
template <int KB, bool VEC_OUT, typename IdxT>
__global__ __launch_bounds__(kWave) void bucket_quads(SelectArgs a) {
  constexpr int kStride = kQuadWidth + 4;  // LDS floats per bucket (skew of 16 bytes)
  constexpr int kChunks = kQuadWidth / 4;  // 16-byte chunks per bucket
  constexpr int kLoads = kQuadGroup * kChunks / kWave;  // chunks per lane
  static_assert(kWave / kChunks == 2, "a load covers two buckets");
  static_assert(KB % 4 == 0, "survivor slots run in chunks of four");
  __shared__ u32x4 stage[kQuadGroup * kStride / 4];
  // The output assembly area at the start of the stage: kOutEntries value
  // words and a spare one, then the indices (bytes or words) from word
  // kOutIdx, and their spare entry.
  constexpr int kOutEntries = kQuadGroup * KB;
  constexpr int kOutIdx = kOutEntries + 4;
  constexpr int kOutWords = kOutIdx + (sizeof(IdxT) == 1 ? kOutEntries / 4 + 4 : kOutEntries + 4);
  static_assert(kOutEntries % 64 == 0 || kOutEntries <= 256, "one store per array");
  static_assert(kOutWords <= kQuadGroup * kStride, "assembly fits the stage");
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  const int bl = lane & (kQuadGroup - 1);  // bucket within the group
  const int h = lane / kQuadGroup;         // quarter
  const int w = a.m, kb = a.k;
  const int64_t groups = (a.n + kQuadGroup - 1) / kQuadGroup;
  int64_t grp = blockIdx.x;
  if (grp >= groups) return;
  auto live_of = [&](int64_t g) {
    const int64_t rest = a.n - g * kQuadGroup;
    return rest < kQuadGroup ? static_cast<int>(rest) : kQuadGroup;
  };
  // Load i covers buckets 2i and 2i + 1 (lane / 32 picks the bucket, lane
  // mod 32 the chunk) through a resource of its own that starts at bucket
  // 2i and ends at the group's end: every load takes the same lane offset,
  // and the bounds check drops chunks past the group's buckets (they read
  // zeros). Chunks past a bucket's end (w < 128) belong to the next bucket
  // and are not written to LDS below.
  const int load_off = ((lane / kChunks) * w + 4 * (lane % kChunks)) * 4;
  auto load = [&](int64_t g, u32x4 (&q)[kLoads]) {
    const float* x0 = a.x + g * kQuadGroup * w;
    const int bytes = live_of(g) * w * 4;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int skip = i * 8 * w;
      const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float*>(x0) + 2 * i * w, 0, bytes > skip ? bytes - skip : 0, kRsrcWord3);
      q[i] = __builtin_amdgcn_raw_buffer_load_b128(rx, load_off, 0, kLoadPolicy);
    }
  };
  u32x4 q[kLoads];
  load(grp, q);
  // Places past w of every LDS bucket row hold -inf for the whole kernel
  // (the staging below writes places < w only), which takes them out of
  // every comparison (the inputs are finite). Written after the first
  // loads are issued, so that they do not wait behind it.
  if (w < kQuadWidth) {
    constexpr u32x4 kNegInf = {0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u};
    for (int i = lane; i < kQuadGroup * kStride / 4; i += kWave) stage[i] = kNegInf;
  }
  // Load i lands at stage chunk i * (2 * kStride / 4) + (lane / 32) *
  // kStride / 4 + lane mod 32: each half-wave writes 512 consecutive bytes.
  const int stage_at = (lane / kChunks) * (kStride / 4) + (lane % kChunks);
  // Sums over the bucket's four quarters of a per-lane count: the count of
  // the quarters before this lane's, and the bucket's total (see
  // swap_rows: lo holds the even quarter of each pair, then the first half).
  auto quarter_prefix = [&](int c, int& before, int& total) {
    uint32_t lo, hi;
    swap_rows<16>(static_cast<uint32_t>(c), lo, hi);
    const int pair = static_cast<int>(lo + hi);
    uint32_t lo2, hi2;
    swap_rows<32>(static_cast<uint32_t>(pair), lo2, hi2);
    before = ((h & 1) ? static_cast<int>(lo) : 0) + ((h & 2) ? static_cast<int>(lo2) : 0);
    total = static_cast<int>(lo2 + hi2);
  };
  const uint32_t nb = static_cast<uint32_t>(a.buckets);
  for (;;) {
    const int64_t g0 = grp * kQuadGroup;
    const int live = live_of(grp);
    if (w == kQuadWidth && live == kQuadGroup) {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) stage[i * (2 * kStride / 4) + stage_at] = q[i];
    } else {
#pragma unroll
      for (int i = 0; i < kLoads; ++i) {
        const int bkt = 2 * i + lane / kChunks;
        if (4 * (lane % kChunks) < w && bkt < live) stage[i * (2 * kStride / 4) + stage_at] = q[i];
      }
    }
    // LDS operations of one wave complete in issue order; the barriers keep
    // the compiler from moving the reads above the writes (and, at the
    // loop's end, the next group's writes above this group's reads).
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
    const int64_t next = grp + gridDim.x;
    if (next < groups) load(next, q);
    // The lane's quarter: 16 lanes of one quarter read 16 buckets whose
    // rows are 528 bytes apart, so the 16-byte reads fall in 16 different
    // bank groups.
    const float* row = reinterpret_cast<const float*>(stage) + bl * kStride + kQuarter * h;
    float v[kQuarter];
#pragma unroll
    for (int j = 0; j < kQuarter; j += 4) {
      const u32x4 e = *reinterpret_cast<const u32x4*>(row + j);
      v[j] = __uint_as_float(e.x);
      v[j + 1] = __uint_as_float(e.y);
      v[j + 2] = __uint_as_float(e.z);
      v[j + 3] = __uint_as_float(e.w);
    }
    // The KB largest values of the quarter, largest first. Up to 8: by
    // median-of-three insertion (KB instructions per place). 16: two sorted
    // batches of 16 (odd-even merge sort, 63 compare-exchanges each) merged.
    float tv[KB];
    if constexpr (KB >= 16) {
      float bt[KB];
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        tv[i] = v[i];
        bt[i] = v[KB + i];
      }
      sort_desc(tv);
      sort_desc(bt);
      merge_top_desc(tv, bt);
    } else {
#pragma unroll
      for (int i = 0; i < KB; ++i) tv[i] = -__builtin_inff();
#pragma unroll
      for (int j = 0; j < kQuarter; ++j) {
        const float x = v[j];
#pragma unroll
        for (int i = KB - 1; i > 0; --i) tv[i] = __builtin_amdgcn_fmed3f(tv[i - 1], x, tv[i]);
        tv[0] = fmaxf(tv[0], x);
      }
    }
    // The bucket's KB largest values: merged with the other quarter of the
    // half, then with the other half. The lists are exchanged with lane
    // swaps; each lane of a pair merges the two lists in one orientation or
    // the other, which yields the same sorted list.
    {
      float lo[KB], hi[KB];
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        uint32_t a, b;
        swap_rows<16>(__float_as_uint(tv[i]), a, b);
        lo[i] = __uint_as_float(a);
        hi[i] = __uint_as_float(b);
      }
      merge_top_desc(lo, hi);
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        uint32_t a, b;
        swap_rows<32>(__float_as_uint(lo[i]), a, b);
        tv[i] = __uint_as_float(a);
        hi[i] = __uint_as_float(b);
      }
      merge_top_desc(tv, hi);
    }
    // The kb-th largest value of the bucket and how many of the kb largest
    // equal it.
    float thr = tv[0];
#pragma unroll
    for (int i = 1; i < KB; ++i) thr = i < kb ? tv[i] : thr;
    int need_eq = 0;
#pragma unroll
    for (int i = 0; i < KB; ++i) need_eq += (i < kb && tv[i] == thr) ? 1 : 0;
    // Places of the quarter at or above thr: place j at bit 31 - j. The
    // quarter is read from the stage again: holding it across the merges
    // would take 32 more registers (and a wave per SIMD).
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < kQuarter; j += 4) {
      const u32x4 e = *reinterpret_cast<const u32x4*>(row + j);
      v[j] = __uint_as_float(e.x);
      v[j + 1] = __uint_as_float(e.y);
      v[j + 2] = __uint_as_float(e.z);
      v[j + 3] = __uint_as_float(e.w);
    }
    const float thr_s = zero_as_minus(thr);
    uint32_t below = 0;
#pragma unroll
    for (int j = 0; j < kQuarter; ++j) below = shift_in_lt(below, v[j], thr_s);
    uint32_t keep = ~below;
    int count = __builtin_popcount(keep);
    int base, total;
    quarter_prefix(count, base, total);
    if (__builtin_amdgcn_ballot_w64(total > kb) != 0) {
      // Surplus ties at thr: keep every place above it and the need_eq
      // lowest-column places equal to it, lower quarters first.
      uint32_t equal = 0;
#pragma unroll
      for (int j = 0; j < kQuarter; ++j) shift_in_eq(equal, v[j], thr);
      keep &= ~equal;
      int eq_before, eq_total;
      quarter_prefix(__builtin_popcount(equal), eq_before, eq_total);
      const int quota = need_eq - eq_before;
#pragma unroll
      for (int i = 0; i < KB; ++i) {
        const uint32_t top = equal != 0u ? 0x80000000u >> __builtin_clz(equal) : 0u;
        const uint32_t take = i < quota ? top : 0u;
        keep |= take;
        equal ^= take;
      }
      count = __builtin_popcount(keep);
      quarter_prefix(count, base, total);
    }
    const uint32_t r0 = g0 < 0x100000000LL ? static_cast<uint32_t>(g0) % nb
                                           : static_cast<uint32_t>(g0 % a.buckets);
    const uint32_t first =
        ((r0 + static_cast<uint32_t>(bl)) % nb) * static_cast<uint32_t>(w) + kQuarter * h;
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
        a.out_val + g0 * kb, 0, live * kb * 4, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t ri = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<IdxT*>(a.out_idx) + g0 * kb, 0,
        live * kb * static_cast<int>(sizeof(IdxT)), kRsrcWord3);
    // The values of the lane's survivors, lowest column first (the LDS
    // reads issued together rather than one wait per survivor).
    // Slots run in chunks of four, and a chunk no lane of the wave needs
    // is skipped (a lane keeps kb / 4 places of its quarter on average).
    auto chunk_needed = [&](int c4) {
      return c4 == 0 || __builtin_amdgcn_ballot_w64(count > c4) != 0;
    };
    uint32_t xs[KB];
    {
      uint32_t k2 = keep;
#pragma unroll
      for (int c4 = 0; c4 < KB; c4 += 4) {
        if (!chunk_needed(c4)) break;
#pragma unroll
        for (int i = c4; i < c4 + 4; ++i) {
          const int c = k2 != 0u ? __builtin_clz(k2) : 0;
          xs[i] = __float_as_uint(row[c]);
          k2 &= ~(0x80000000u >> c);
        }
      }
    }
    // The group's outputs are one contiguous stretch of live * kb entries
    // (at most 1 KB of values): they are assembled in the stage (free once
    // the reads above are done; LDS operations of one wave complete in
    // issue order) and stored with one coalesced store per array. Stored
    // straight from each lane, every entry was a 4-byte (and a 1-byte)
    // store of its own: 32 store instructions per group, each writing 64
    // scattered words, which kept the texture address unit busy 70% of the
    // time. Entries past a lane's survivors write the spare entry; the
    // columns are found again rather than kept in registers.
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
    uint32_t* const out_val = reinterpret_cast<uint32_t*>(stage);
#pragma unroll
    for (int c4 = 0; c4 < KB; c4 += 4) {
      if (!chunk_needed(c4)) break;
#pragma unroll
      for (int i = c4; i < c4 + 4; ++i) {
        const int c = keep != 0u ? __builtin_clz(keep) : 0;
        keep &= ~(0x80000000u >> c);
        const int e = i < count ? bl * kb + base + i : kOutEntries;
        out_val[e] = xs[i];
        if constexpr (sizeof(IdxT) == 1)
          reinterpret_cast<uint8_t*>(out_val + kOutIdx)[e] = static_cast<uint8_t>(first + c);
        else
          out_val[kOutIdx + e] = first + c;
      }
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
    // Lane l stores entries 4l .. 4l + 3 of each array (16-byte value
    // stores when the output is 16-byte aligned, else four words); the
    // resources' bounds drop entries past live * kb.
    {
      const u32x4 vals = reinterpret_cast<const u32x4*>(out_val)[lane];
      if constexpr (VEC_OUT) {
        __builtin_amdgcn_raw_buffer_store_b128(vals, rv, lane * 16, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b32(vals.x, rv, lane * 16, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(vals.y, rv, lane * 16 + 4, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(vals.z, rv, lane * 16 + 8, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(vals.w, rv, lane * 16 + 12, 0, 0);
      }
      if constexpr (sizeof(IdxT) == 1) {
        const uint32_t idx4 = out_val[kOutIdx + lane];
        // The bounds check drops a word that is only partly in range: the
        // lane holding the last entries of a stretch whose length is not a
        // multiple of 4 stores them byte by byte.
        const int n_idx = live * kb;
        if (VEC_OUT && 4 * lane + 4 <= n_idx) {
          __builtin_amdgcn_raw_buffer_store_b32(idx4, ri, lane * 4, 0, 0);
        } else {
#pragma unroll
          for (int b = 0; b < 4; ++b)
            __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(idx4 >> (8 * b)), ri,
                                                 lane * 4 + b, 0, 0);
        }
      } else {
        const u32x4 idx = reinterpret_cast<const u32x4*>(out_val + kOutIdx)[lane];
        if constexpr (VEC_OUT) {
          __builtin_amdgcn_raw_buffer_store_b128(idx, ri, lane * 16, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b32(idx.x, ri, lane * 16, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(idx.y, ri, lane * 16 + 4, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(idx.z, ri, lane * 16 + 8, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(idx.w, ri, lane * 16 + 12, 0, 0);
        }
      }
    }
    // Short buckets: the assembly overwrote places past w of the first
    // bucket rows, which must read -inf.
    if (w < kQuadWidth) {
      __builtin_amdgcn_wave_barrier();
      constexpr u32x4 kNegInf = {0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u};
      for (int i = lane; i < kOutWords / 4; i += kWave) stage[i] = kNegInf;
    }
    if (next >= groups) break;
    grp = next;
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
  }
}

template <bool VEC_OUT, typename IdxT>
RowsKernel pick_quad_kb(int kb) {
  if (kb <= 4) return bucket_quads<4, VEC_OUT, IdxT>;
  if (kb <= 8) return bucket_quads<8, VEC_OUT, IdxT>;
  return bucket_quads<16, VEC_OUT, IdxT>;
}

template <typename IdxT>
RowsKernel pick_quad(const SelectArgs& a) {
  const bool vec_out = ((reinterpret_cast<uintptr_t>(a.out_val) |
                         reinterpret_cast<uintptr_t>(a.out_idx)) & 15) == 0;
  return vec_out ? pick_quad_kb<true, IdxT>(a.k) : pick_quad_kb<false, IdxT>(a.k);
}

template <int W, bool VEC, typename IdxT>
RowsKernel pick_kb(int kb) {
  if (kb <= 1) return bucket_lanes<W, 1, VEC, IdxT>;
  if (kb <= 2) return bucket_lanes<W, 2, VEC, IdxT>;
  if (kb <= 4) return bucket_lanes<W, 4, VEC, IdxT>;
  return bucket_lanes<W, 8, VEC, IdxT>;
}

template <bool VEC, typename IdxT>
RowsKernel pick_w(int w, int kb) {
  if (w <= 8) return pick_kb<8, VEC, IdxT>(kb);
  if (w <= 16) return pick_kb<16, VEC, IdxT>(kb);
  if (w <= 32) return pick_kb<32, VEC, IdxT>(kb);
  return pick_kb<64, VEC, IdxT>(kb);
}

template <typename IdxT>
RowsKernel pick(int w, int kb, bool vec) {
  return vec ? pick_w<true, IdxT>(w, kb) : pick_w<false, IdxT>(w, kb);
}

}  // namespace bucket_detail

bool bucket_lanes_supported(const float* x, int width, int kb) {
  if (width <= kLaneBucketWidth) return kb <= kLaneBucketSurvivors;
  return width <= kQuadBucketWidth && kb <= kQuadBucketSurvivors && width % 4 == 0 &&
         (reinterpret_cast<uintptr_t>(x) & 15u) == 0;
}

hipError_t launch_bucket_lanes(const SelectArgs& a, bool u8_index,
                               hipStream_t stream) {
  using namespace bucket_detail;
  const bool vec = a.m % 4 == 0 && (reinterpret_cast<uintptr_t>(a.x) & 15u) == 0;
  const bool quads = a.m > kLaneBucketWidth;
  if (quads && (!vec || a.m > kQuadWidth || a.k > kQuadBucketSurvivors))
    return hipErrorInvalidValue;
  const RowsKernel fn = quads ? (u8_index ? pick_quad<uint8_t>(a) : pick_quad<int32_t>(a))
                              : (u8_index ? pick<uint8_t>(a.m, a.k, vec)
                                          : pick<int32_t>(a.m, a.k, vec));
  const int threads = kLaneWaves * kWave;
  const int per_block = quads ? kQuadGroup : threads;
  int64_t blocks = (a.n + per_block - 1) / per_block;
  // Staged groups (16-byte loads, buckets of more than 16 columns): a
  // persistent grid of what is resident; the waves loop over the groups.
  // Every wave gets the same share of groups, so the single-wave blocks per
  // CU are rounded down to a multiple of the CU's four SIMDs: with 17 (the
  // LDS limit of the 32-column kernel) one SIMD ran five waves, and the
  // whole launch waited for it (measured 3% slower than 16).
  if (vec && a.m > 16 && blocks > 0) {
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return hipErrorInvalidDevice;
    int per_cu = resident_blocks(reinterpret_cast<const void*>(fn), threads, device);
    if (per_cu >= kSimdsPerCu) per_cu -= per_cu % kSimdsPerCu;
    // At most three waves per SIMD, though 16 fit at 32 columns (and fitted
    // the four-lane kernel before its survivor slots ran in chunks): each
    // wave keeps a group (8 KB) of loads in flight, and fewer of them ran
    // faster (one box, us, 16 -> 12 waves per CU: 262,144 x 256 in 2
    // buckets 67.4 -> 66.1, in 8 buckets 58.6 -> 57.9; 1,048,576 x 128,
    // k = 16 135.6 -> 131.9, k = 8 117.9 -> 116.9; 2,097,152 x 32 58.7 ->
    // 57.9; 8 waves: slower on the four-lane kernel).
    per_cu = per_cu < kMaxStagedWavesPerCu ? per_cu : kMaxStagedWavesPerCu;
    const int64_t resident = static_cast<int64_t>(cu_count(device)) * per_cu;
    blocks = blocks < resident ? blocks : resident;
  }
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(fn, dim3(static_cast<uint32_t>(blocks)), dim3(threads), 0,
                     stream, a);
  return hipGetLastError();
}

}  // namespace rtopk
