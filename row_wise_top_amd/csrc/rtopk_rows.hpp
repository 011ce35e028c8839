#pragma once

// Row-wise top-k kernels for gfx950 (CDNA4, wave64): device templates.
// Included by the rtopk_rows_*.hip units, each of which instantiates the
// kernels for a few slot counts (so the units compile in parallel).
//
// Method: RTop-K summary page ("RTop-K: Ultra-Fast Row-Wise Top-K Selection
// for Neural Network Acceleration on GPUs"), section "Approach": per row, a
// search over the value range for a threshold that selects k elements, an
// optional cap on the number of search steps, and a second pass that fills
// the remaining slots from the lower end of the search range. The output is
// the two dense [N, k] arrays (values, column indices) of the compressed
// balanced layout in the MaxK-GNN review, "How MaxK-GNN works".
//
// Mapping. One wave64 owns one row at a time. The row lives in registers:
// lane l, slot s holds column 64*s + l, so each slot is one fully coalesced
// 256-byte load and the order of columns is (slot, lane). A count of
// elements >= t is one v_cmp per slot producing a 64-bit lane mask, summed
// with scalar popcounts; nothing is re-read from memory during the search.
// Compaction in column order needs only the scalar prefix over earlier slots
// plus the lane's rank inside its slot's mask (mbcnt).
//
// Each wave takes rows in groups and issues the loads of its next rows
// before working on the current one, so HBM reads overlap the search.
//
// Two searches share this skeleton:
//  * capped (rtopk_select): the bisection of the summary page, step for step
//    as specified in rtopk.h, from [min, max] of the row;
//  * exact (rtopk_select_exact): any sequence of thresholds is allowed as
//    long as the result is the exact top-k, so the thresholds are chosen to
//    need few counts. The first one comes from the row's mean and standard
//    deviation under a normal model, aimed at a count a little above k. Once
//    a count lands in (k, W] (W = 64*QC), the elements at or above that
//    threshold are the only candidates left; they are compacted through LDS
//    into QC slots in column order, so every further count costs QC compares
//    instead of Q. Newton steps with the model's density follow, then a
//    "snap" to the largest candidate below the upper bound resolves ties.
//    Bisection of the integer order keys (at most 32 counts) bounds every
//    case the model handles badly. The model only picks thresholds; the
//    result never depends on it.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "rtopk_internal.h"

namespace rtopk {
namespace rows_detail {

constexpr float kInf = __builtin_inff();
// Word 3 of a gfx9 buffer resource for untyped 32-bit access (data format 32).
constexpr int kRsrcWord3 = 0x00020000;
// Cache policy of the row loads (gfx950 encoding, bit 1 = non-temporal).
constexpr int kLoadNT = 2;

// ---------------------------------------------------------------------------
// Wave-level primitives
// ---------------------------------------------------------------------------

// Number of set bits of `mask` at lanes below the calling lane, plus `acc`.
__device__ __forceinline__ uint32_t rank_below(uint64_t mask, uint32_t acc = 0u) {
  return __builtin_amdgcn_mbcnt_hi(
      static_cast<uint32_t>(mask >> 32),
      __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), acc));
}

__device__ __forceinline__ uint64_t ballot(bool p) {
  return __builtin_amdgcn_ballot_w64(p);
}

__device__ __forceinline__ int popc(uint64_t m) { return __popcll(m); }

// (bit `lane` of mask) ? a : b, as one v_cndmask. Written out because the
// compiler turns a select whose operand is only needed on one side into an
// exec-masked region (two scalar instructions to save and restore exec).
__device__ __forceinline__ uint32_t lane_select(uint64_t mask, uint32_t a,
                                                uint32_t b) {
  uint32_t r;
  asm("v_cndmask_b32_e64 %0, %2, %1, %3" : "=v"(r) : "v"(a), "v"(b), "s"(mask));
  return r;
}

// Cross-lane read through DPP, all rows and banks enabled. A lane whose
// source does not exist (row 0 for the row broadcasts) reads 0 (bound_ctrl);
// the reductions below only use lane 63, whose sources always exist.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                         0xf, 0xf, true));
}

// DPP controls (gfx9 encoding).
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;
constexpr int kRowBcast15 = 0x142;    // lane 15 of each row -> next row
constexpr int kRowBcast31 = 0x143;    // lane 31 -> rows 2 and 3

__device__ __forceinline__ float lane63(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Two wave-wide reductions, interleaved so that each DPP step of one hides
// the read-after-write wait of the other. Op is min, max or +. After the
// four in-row steps every lane holds its row's result; the two broadcasts
// then accumulate rows 0..3 into lane 63.
struct OpMin {
  __device__ static float f(float a, float b) { return fminf(a, b); }
};
struct OpMax {
  __device__ static float f(float a, float b) { return fmaxf(a, b); }
};
struct OpAdd {
  __device__ static float f(float a, float b) { return a + b; }
};

template <class A, class B>
__device__ __forceinline__ void wave_reduce2(float& a, float& b) {
  a = A::f(a, dpp<kQuadSwap1>(a));
  b = B::f(b, dpp<kQuadSwap1>(b));
  a = A::f(a, dpp<kQuadSwap2>(a));
  b = B::f(b, dpp<kQuadSwap2>(b));
  a = A::f(a, dpp<kRowHalfMirror>(a));
  b = B::f(b, dpp<kRowHalfMirror>(b));
  a = A::f(a, dpp<kRowMirror>(a));
  b = B::f(b, dpp<kRowMirror>(b));
  a = A::f(a, dpp<kRowBcast15>(a));
  b = B::f(b, dpp<kRowBcast15>(b));
  a = A::f(a, dpp<kRowBcast31>(a));
  b = B::f(b, dpp<kRowBcast31>(b));
  a = lane63(a);
  b = lane63(b);
}

__device__ __forceinline__ float wave_max(float a) {
  a = fmaxf(a, dpp<kQuadSwap1>(a));
  a = fmaxf(a, dpp<kQuadSwap2>(a));
  a = fmaxf(a, dpp<kRowHalfMirror>(a));
  a = fmaxf(a, dpp<kRowMirror>(a));
  a = fmaxf(a, dpp<kRowBcast15>(a));
  a = fmaxf(a, dpp<kRowBcast31>(a));
  return lane63(a);
}

// ---------------------------------------------------------------------------
// Row in registers
// ---------------------------------------------------------------------------

// Load a row into slots. FULL: the row length is exactly 64*Q. Otherwise the
// row is read through a buffer resource of exactly m floats: positions past
// the end read 0 (mask_tail() then makes them -inf), and every slot's load
// is the lane's offset plus a constant, so no per-slot address stays live
// (with clamped addresses the compiler kept one per slot across the row
// loop: 256 VGPRs and thousands of spill instructions at 128 slots). The
// input is read once: non-temporal loads keep it from displacing other
// lines in the caches (measured: the memory-only floor of the 262,144 x 256
// selection drops from 54 to 49.5 us).
template <int Q, bool FULL>
__device__ __forceinline__ void load_row(const float* __restrict__ row, int m,
                                         int lane, float (&v)[Q]) {
  if constexpr (FULL) {
#pragma unroll
    for (int s = 0; s < Q; ++s) v[s] = __builtin_nontemporal_load(row + s * kWave + lane);
  } else {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(row), 0, m * 4, kRsrcWord3);
#pragma unroll
    for (int s = 0; s < Q; ++s)
      v[s] = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(r, lane * 4, s * kWave * 4, kLoadNT));
  }
}

// Positions past the end become -inf: no count and no selection test picks
// them (every threshold used is finite or the bracket end +-inf, and the
// tests are x >= t with t > -inf). The row length goes through an empty asm
// so that the per-slot tests are made here, once per row, and not hoisted
// out of the row loop as one live lane mask per slot.
template <int Q, bool FULL>
__device__ __forceinline__ void mask_tail(int m, int lane, float (&v)[Q]) {
  if (FULL) return;
  int mo = m;
  asm volatile("" : "+s"(mo));
#pragma unroll
  for (int s = 0; s < Q; ++s) {
    if (!(s * kWave + lane < mo)) v[s] = -kInf;
  }
}

// #{elements >= t}: one compare per slot, scalar popcounts.
template <int S>
__device__ __forceinline__ int count_ge(const float (&v)[S], float t) {
  int c = 0;
#pragma unroll
  for (int s = 0; s < S; ++s) c += popc(ballot(v[s] >= t));
  return c;
}

// Order-preserving map from floats to int32 (-0 and +0 both map to 0,
// +-inf map to +-0x7f800000) and its inverse.
__device__ __forceinline__ int32_t order_key(float f) {
  const int32_t b = __float_as_int(f);
  return b >= 0 ? b : static_cast<int32_t>(0x80000000u - static_cast<uint32_t>(b));
}

__device__ __forceinline__ float key_value(int32_t key) {
  const uint32_t b = key >= 0 ? static_cast<uint32_t>(key)
                              : 0x80000000u - static_cast<uint32_t>(key);
  return __int_as_float(static_cast<int32_t>(b));
}

// ---------------------------------------------------------------------------
// Emission. Every emission writes exactly k entries, in column order.
// `col(s)` gives the column held by slot s of the calling lane.
//
// The two output rows are addressed as buffer resources whose size is the
// row's k entries. A buffer store at an offset past that size is discarded
// by the hardware, so every lane stores and the lanes not selected use a
// position past the end: the stores need no exec-mask changes and the
// compiler's wait counts stay exact.
// ---------------------------------------------------------------------------


// Output position of a lane that stores nothing: past any row end, and times
// four still a valid 32-bit offset.
constexpr uint32_t kDropPos = 1u << 28;
// Cache policy of the stores (gfx950 encoding, bit 1 = non-temporal). Values,
// 32-bit indices and dense rows stream out non-temporally; one-byte index
// rows (often a fraction of a 128-byte line) keep the default policy so
// that the rows of a line merge in L2 before they are written back.
constexpr int kStoreNT = 2;

// Mode::kMaxk: every survivor is also written, as value bits, to its column
// of the wave's LDS copy of the dense row (zeroed before the row and stored
// after it); lanes not selected write their spare word instead.
// Mode::kBucket: emitted columns are offset by the bucket's first column.
template <typename IdxT, Mode MODE>
struct OutRow {
  __amdgpu_buffer_rsrc_t val;
  __amdgpu_buffer_rsrc_t idx;
  uint32_t* dense;   // kMaxk only: the LDS row (plus one spare word per lane)
  uint32_t spare;    // kMaxk only: this lane's spare word
  int col_base;      // kBucket only: column of the bucket's first element

  __device__ __forceinline__ OutRow(float* ov, IdxT* oi, int k,
                                    uint32_t* dense_row, uint32_t spare_word,
                                    int first_col)
      : val(__builtin_amdgcn_make_buffer_rsrc(ov, 0, k * 4, kRsrcWord3)),
        idx(__builtin_amdgcn_make_buffer_rsrc(
            oi, 0, k * static_cast<int>(sizeof(IdxT)), kRsrcWord3)),
        dense(dense_row),
        spare(spare_word),
        col_base(first_col) {}

  // Entry `pos` of the row: value bits and column (positions past the row's
  // k entries are dropped by the buffer bounds). Used by StagedOut.
  __device__ __forceinline__ void store_entry(uint32_t pos, uint32_t xbits,
                                              uint32_t col) const {
    __builtin_amdgcn_raw_buffer_store_b32(xbits, val, static_cast<int>(pos * 4u), 0,
                                          kStoreNT);
    if constexpr (sizeof(IdxT) == 1) {
      __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(col), idx,
                                           static_cast<int>(pos), 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b32(col, idx, static_cast<int>(pos * 4u), 0,
                                            kStoreNT);
    }
  }

  // Lanes whose bit of `msk` is set emit (x, col) as entry `rank` of the row;
  // the others store nothing.
  __device__ __forceinline__ void put(uint64_t msk, uint32_t rank, float x,
                                      int col) const {
    const uint32_t pos = lane_select(msk, rank, kDropPos);
    if constexpr (MODE == Mode::kMaxk)
      dense[lane_select(msk, static_cast<uint32_t>(col), spare)] = __float_as_uint(x);
    if constexpr (MODE == Mode::kBucket) col += col_base;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), val,
                                          static_cast<int>(pos * 4u), 0, kStoreNT);
    if constexpr (sizeof(IdxT) == 1) {
      __builtin_amdgcn_raw_buffer_store_b8(static_cast<uint8_t>(col), idx,
                                           static_cast<int>(pos), 0, 0);
    } else {
      __builtin_amdgcn_raw_buffer_store_b32(static_cast<uint32_t>(col), idx,
                                            static_cast<int>(pos * 4u), 0, kStoreNT);
    }
  }
};

// The second pass: the first k (by column) of A = {x >= hi}, then of
// B = {lo <= x < hi}, written in column order. The caller passes
// nA = #{x >= hi} and guarantees #{x >= lo} >= k.
//  * nA >= k (only possible in the capped search, when the bracket never
//    left the row maximum): the survivors are the first k of A. Every element
//    of A is stored at its rank; ranks past k fall outside the output row's
//    buffer resource and the hardware drops them.
//  * nA < k: all of A, and the elements of B whose rank among B (in column
//    order) is below k - nA.
template <int S, typename Out, typename ColFn>
__device__ __forceinline__ void emit_fill(const float (&v)[S], ColFn col,
                                          float lo, float hi, int k, int nA,
                                          const Out& out) {
  if constexpr (S > 32) {
    // As in emit_ge: no lane masks kept alive from earlier counts.
    asm volatile("" : "+v"(lo));
    asm volatile("" : "+v"(hi));
  }
  if (nA >= k) {
    // The exact searches reach this only with nA == k (no rank is dropped,
    // so the MaxK dense row gets exactly the k survivors).
    uint32_t base = 0;
#pragma unroll
    for (int s = 0; s < S; ++s) {
      const uint64_t mA = ballot(v[s] >= hi);
      out.put(mA, rank_below(mA, base), v[s], col(s));
      base += popc(mA);
    }
    return;
  }
  const uint32_t need = static_cast<uint32_t>(k - nA);
  uint32_t base = 0, baseB = 0;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const uint64_t mA = ballot(v[s] >= hi);
    const uint64_t mB = ballot(v[s] >= lo) & ~mA;
    const uint64_t keepB = ballot(rank_below(mB, baseB) < need) & mB;
    const uint64_t mS = mA | keepB;
    out.put(mS, rank_below(mS, base), v[s], col(s));
    baseB += popc(mB);
    base += popc(mS);
  }
}

// ---------------------------------------------------------------------------
// Exact search (rtopk_select_exact).
// Bracket invariant: #{x >= lo} = clo >= k > chi = #{x >= hi}, with
// lo = -inf and hi = +inf allowed at the start. Every count at a threshold t
// gives a valid new bound whether or not t lies inside the bracket (c > k:
// lo = t; c < k: hi = t), so the pivots need no bounds check. A count of
// exactly k at t ends the search (the result is {x >= t}); otherwise the
// search ends on the k-th largest value v, and the result is {x > v} plus the
// lowest columns holding v.
// ---------------------------------------------------------------------------

// Full-row Newton steps before the order-key bisection takes over.
constexpr int kRowSteps = 4;
// Newton steps, then snaps, on the compacted candidates.
constexpr int kCandSteps = 5;
constexpr int kCandSnaps = 4;

__device__ __forceinline__ float wave_min(float a) {
  a = fminf(a, dpp<kQuadSwap1>(a));
  a = fminf(a, dpp<kQuadSwap2>(a));
  a = fminf(a, dpp<kRowHalfMirror>(a));
  a = fminf(a, dpp<kRowMirror>(a));
  a = fminf(a, dpp<kRowBcast15>(a));
  a = fminf(a, dpp<kRowBcast31>(a));
  return lane63(a);
}

__device__ __forceinline__ float wave_sum(float a) {
  a += dpp<kQuadSwap1>(a);
  a += dpp<kQuadSwap2>(a);
  a += dpp<kRowHalfMirror>(a);
  a += dpp<kRowMirror>(a);
  a += dpp<kRowBcast15>(a);
  a += dpp<kRowBcast31>(a);
  return lane63(a);
}

// Wave-wide reductions of a group's values, four at a time (N a multiple
// of four, all results uniform). gfx950's lane swaps fold two values per
// instruction pair: permlane32_swap(a, b) leaves a's lanes 0-31 and b's
// lanes 0-31 in one register, a's lanes 32-63 and b's lanes 32-63 in the
// other, so one op reduces a to 32 lanes (0-31) and b to 32 lanes (32-63);
// permlane16_swap then does the same for 16-lane rows, leaving four values
// reduced to one 16-lane row each (value 0 in row 0, 2 in row 1, 1 in row 2,
// 3 in row 3). Four in-row DPP steps finish all four at once. Per four
// values: 3 swaps, 7 ops and 4 reads of a lane, against 28 instructions as
// four separate reductions. The sums come out in another order than
// wave_sum's; min and max are exact in any order.
template <class Op>
__device__ __forceinline__ float fold_pair32(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b),
                                                  false, false);
  return Op::f(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <class Op>
__device__ __forceinline__ float fold_pair16(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b),
                                                  false, false);
  return Op::f(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// The reductions of N values (N % 4 == 0) with one op, in steps, so that
// the steps of several of them can be interleaved (each hides the waits of
// the others).
template <class Op, int N>
struct GroupReduce {
  static_assert(N % 4 == 0, "groups of four values");
  static constexpr int G = N / 4;
  float (&a)[N];
  float f[2 * G];

  // 64 -> 32 lanes, then 32 -> 16 lanes.
  __device__ __forceinline__ void fold32() {
#pragma unroll
    for (int g = 0; g < 2 * G; ++g) f[g] = fold_pair32<Op>(a[2 * g], a[2 * g + 1]);
  }
  __device__ __forceinline__ void fold16() {
#pragma unroll
    for (int g = 0; g < G; ++g) f[g] = fold_pair16<Op>(f[2 * g], f[2 * g + 1]);
  }
  template <int C>
  __device__ __forceinline__ void in_row() {
#pragma unroll
    for (int g = 0; g < G; ++g) f[g] = Op::f(f[g], dpp<C>(f[g]));
  }
  __device__ __forceinline__ void finish() {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      a[4 * g] = lane_value(f[g], 0);
      a[4 * g + 1] = lane_value(f[g], 32);
      a[4 * g + 2] = lane_value(f[g], 16);
      a[4 * g + 3] = lane_value(f[g], 48);
    }
  }
};

template <class... R>
__device__ __forceinline__ void run_group_reduce(R&... r) {
  (r.fold32(), ...);
  (r.fold16(), ...);
  (r.template in_row<kQuadSwap1>(), ...);
  (r.template in_row<kQuadSwap2>(), ...);
  (r.template in_row<kRowHalfMirror>(), ...);
  (r.template in_row<kRowMirror>(), ...);
  (r.finish(), ...);
}

// N wave-wide sums (N % 4 == 0).
template <int N>
__device__ __forceinline__ void wave_sum_n(float (&a)[N]) {
  GroupReduce<OpAdd, N> s{a};
  run_group_reduce(s);
}

// N pairs of wave-wide reductions (minimum, maximum; N % 4 == 0).
template <int N>
__device__ __forceinline__ void wave_minmax_n(float (&mn)[N], float (&mx)[N]) {
  GroupReduce<OpMin, N> a{mn};
  GroupReduce<OpMax, N> b{mx};
  run_group_reduce(a, b);
}

// N triples of wave-wide reductions (minimum, maximum, sum; N % 4 == 0).
template <int N>
__device__ __forceinline__ void wave_minmaxsum_n(float (&mn)[N], float (&mx)[N],
                                                 float (&sm)[N]) {
  GroupReduce<OpMin, N> a{mn};
  GroupReduce<OpMax, N> b{mx};
  GroupReduce<OpAdd, N> c{sm};
  run_group_reduce(a, b, c);
}

// The float right after f in the order of order_key.
__device__ __forceinline__ float next_float(float f) {
  return key_value(order_key(f) + 1);
}

// Every element >= t (the caller has counted exactly k), in column order.
// The lane masks come straight from the compares and select the positions.
template <int S, typename Out, typename ColFn>
__device__ __forceinline__ void emit_ge(const float (&v)[S], ColFn col,
                                        float t, const Out& out) {
  // Long rows: recompute the compares rather than let the compiler keep the
  // lane masks of the count that found t alive (one SGPR pair per slot,
  // spilled at 128 slots).
  if constexpr (S > 32) asm volatile("" : "+v"(t));
  uint32_t base = 0;
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const uint64_t msk = ballot(v[s] >= t);
    out.put(msk, rank_below(msk, base), v[s], col(s));
    base += popc(msk);
  }
}

// Order-key bisection until a count equals k or lo, hi are adjacent floats
// (at most 32 counts), then the emission.
template <int S, typename Out, typename ColFn>
__device__ __forceinline__ void finish_by_keys(const float (&v)[S], ColFn col,
                                               int k, float lo, float hi,
                                               int chi, const Out& out) {
  int32_t klo = order_key(lo);
  int32_t khi = order_key(hi);
#pragma unroll 1
  for (;;) {
    const uint32_t width = static_cast<uint32_t>(khi) - static_cast<uint32_t>(klo);
    if (width <= 1u) break;
    const int32_t kmid =
        static_cast<int32_t>(static_cast<uint32_t>(klo) + (width >> 1));
    const float t = key_value(kmid);
    const int c = count_ge(v, t);
    if (c == k) {
      emit_ge(v, col, t, out);
      return;
    }
    const bool up = c > k;
    klo = up ? kmid : klo;
    khi = up ? khi : kmid;
    chi = up ? chi : c;
  }
  emit_fill(v, col, key_value(klo), key_value(khi), k, chi, out);
}

// Snaps, then order-key bisection, on the candidates once the Newton steps
// have not hit k exactly. Each snap settles one distinct value: from above,
// u = largest candidate below hi is the k-th largest iff #{x >= u} >= k;
// from below, u = smallest candidate >= lo is iff #{x > u} <= k. The side
// with fewer values to settle is taken.
template <int QC, typename Out, typename ColFn>
__device__ __forceinline__ void settle_candidates(const float (&cv)[QC],
                                                  ColFn col, int k, float lo,
                                                  int clo, float hi, int chi,
                                                  const Out& out) {
#pragma unroll 1
  for (int it = 0; it < kCandSnaps; ++it) {
    const int need = k - chi;           // survivors still to take from [lo, hi)
    const int span = clo - chi;         // candidates in [lo, hi)
    if (need <= span - need + 1) {
      float u = -kInf;
#pragma unroll
      for (int s = 0; s < QC; ++s) u = fmaxf(u, cv[s] < hi ? cv[s] : -kInf);
      u = wave_max(u);
      const int cu = count_ge(cv, u);
      if (cu >= k) {
        emit_fill(cv, col, u, hi, k, chi, out);
        return;
      }
      hi = u;
      chi = cu;
    } else {
      float u = kInf;
#pragma unroll
      for (int s = 0; s < QC; ++s) u = fminf(u, cv[s] >= lo ? cv[s] : kInf);
      u = wave_min(u);
      const float above = next_float(u);
      const int cg = count_ge(cv, above);
      if (cg <= k) {
        emit_fill(cv, col, u, above, k, cg, out);
        return;
      }
      lo = above;
      clo = cg;
    }
  }
  finish_by_keys(cv, col, k, lo, hi, chi, out);
}

// The candidates left after compaction: QC slots in column order (unused
// lanes hold -inf), all elements >= t0, with c0 = #{x >= t0} in (k, 64*QC].
// A fixed number of Newton steps toward k + 1/2 elements runs straight
// through; a count of exactly k ends the row right there (the emission uses
// the compares of that count). Otherwise the row is settled from the bracket
// given by the start and the last step.
template <int QC, typename Out>
__device__ __forceinline__ void exact_candidates(const float (&cv)[QC],
                                                 const int (&ci)[QC], int k,
                                                 float t0, int c0, float h,
                                                 const Out& out) {
  auto col = [&ci](int s) { return ci[s]; };
  // t + (2c - target2) h, as an fma on the count (vector arithmetic only).
  const float h2 = 2.0f * h;
  const float shift = -static_cast<float>(2 * k + 1) * h;
  float t = t0;
  int c = c0;
#pragma unroll
  for (int i = 0; i < kCandSteps; ++i) {
    t = fmaf(static_cast<float>(c), h2, t + shift);
    c = count_ge(cv, t);
    if (c == k) {
      emit_ge(cv, col, t, out);
      return;
    }
  }
  // Both ends are valid bounds (every count is).
  const bool up = c > k;
  settle_candidates<QC>(cv, col, k, up ? t : t0, up ? c : c0, up ? kInf : t,
                        up ? 0 : c, out);
}

// Whether the LDS staging area of a wave has room for a whole row (64*Q
// entries): then a candidate's rank needs no capacity check.
template <int Q>
constexpr bool stage_whole_row() {
  return Q <= 8;
}

// Entries of the staging area that ranks can reach; 64 spare entries (one
// per bank) follow them.
template <int Q, int QC>
constexpr int stage_reach() {
  return stage_whole_row<Q>() ? kWave * Q : kWave * QC;
}

// LDS staging entries per wave for the exact search with QC candidate slots.
template <int Q, int QC>
constexpr int stage_entries() {
  return stage_reach<Q, QC>() + kWave;
}

// Count {x >= t} over the row and, in the same pass, write those elements
// into LDS in column order: value bits at entry e, the column at entry
// E + e, E = stage_entries (two separate words, so no register pairing).
// The staging is only used when the count lands in (k, 64*QC]. Every lane
// writes (no exec-mask changes): lanes whose element is below t, and ranks
// past the reachable part, write the last spare entry (never read), all at
// that one address. Writes of several lanes to one address do not conflict,
// and a slot's candidates take consecutive entries, so a write meets a bank
// conflict only when its candidates' run reaches that entry's bank (with a
// spare entry per lane, 44% of the kernel's LDS cycles were conflicts; a
// spare entry moved per slot to the bank just below the run removes them
// all but costs more instructions than it saves).
template <int Q, int QC>
__device__ __forceinline__ int count_and_stage(const float (&v)[Q], float t,
                                               int lane,
                                               uint32_t* __restrict__ scratch) {
  constexpr uint32_t kE = stage_entries<Q, QC>();
  constexpr uint32_t kSpare = stage_reach<Q, QC>() + kWave - 1;
  uint32_t base = 0;
#pragma unroll
  for (int s = 0; s < Q; ++s) {
    const uint64_t msk = ballot(v[s] >= t);
    uint32_t e = lane_select(msk, rank_below(msk, base), kSpare);
    if constexpr (!stage_whole_row<Q>()) e = min(e, kSpare);
    scratch[e] = __float_as_uint(v[s]);
    scratch[kE + e] = static_cast<uint32_t>(s * kWave + lane);
    base += popc(msk);
  }
  return static_cast<int>(base);
}

// Read back the staged candidates (c of them) into QC slots.
template <int Q, int QC>
__device__ __forceinline__ void read_candidates(const uint32_t* __restrict__ scratch,
                                                int c, int lane, float (&cv)[QC],
                                                int (&ci)[QC]) {
  constexpr int kE = stage_entries<Q, QC>();
  // LDS operations of one wave complete in issue order; the barriers only
  // keep the compiler from moving these reads across the writes.
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < QC; ++j) {
    const int e = j * kWave + lane;
    const float x = __uint_as_float(scratch[e]);
    cv[j] = e < c ? x : -kInf;
    ci[j] = static_cast<int>(scratch[kE + e]);
  }
  __builtin_amdgcn_wave_barrier();
}

// ---------------------------------------------------------------------------
// Capped search (rtopk_select): the specification in rtopk.h, step for step.
// Invariant: #{x >= lo} >= k and (#{x >= hi} < k or hi == row max).
//
// On this GPU the search is bound by instruction issue (vector and scalar
// alike), so each step does only what the specification needs: the
// midpoint, the split test, one count, two selects, and #{x >= hi} for the
// tie fill. Where the count runs decides the cost; the host picks the
// kernel's candidate slots QC by the number of steps:
//  * QC == 0 (one or two steps): every count runs over the row and the tie
//    fill too; narrowing would cost more than the few counts it saves.
//  * QC > 0, stage first: one count at the exact search's first threshold t0 (aimed
//    at the middle of the candidate window) also writes the elements >= t0
//    to LDS. If that count c0 lands in (k, W], W = 64*QC, every specified
//    step counts over those candidates only: for a midpoint >= t0 the count
//    is the row's count, and for one below t0 it is c0 > k, which takes the
//    same branch (lo rises) as the row's count would. The tie fill then runs
//    over the candidates when lo >= t0 (every element >= lo is one of them),
//    else over the row.
//  * otherwise (the first count missed the window): steps over the row until
//    #{x >= lo} fits the window, then the elements >= lo are compacted (every
//    later threshold lies above lo, so counts over them are exact) and the
//    search carries on there.
// ---------------------------------------------------------------------------

// Three wave-wide reductions interleaved (see wave_reduce2).
template <class A, class B, class C>
__device__ __forceinline__ void wave_reduce3(float& a, float& b, float& c) {
  a = A::f(a, dpp<kQuadSwap1>(a));
  b = B::f(b, dpp<kQuadSwap1>(b));
  c = C::f(c, dpp<kQuadSwap1>(c));
  a = A::f(a, dpp<kQuadSwap2>(a));
  b = B::f(b, dpp<kQuadSwap2>(b));
  c = C::f(c, dpp<kQuadSwap2>(c));
  a = A::f(a, dpp<kRowHalfMirror>(a));
  b = B::f(b, dpp<kRowHalfMirror>(b));
  c = C::f(c, dpp<kRowHalfMirror>(c));
  a = A::f(a, dpp<kRowMirror>(a));
  b = B::f(b, dpp<kRowMirror>(b));
  c = C::f(c, dpp<kRowMirror>(c));
  a = A::f(a, dpp<kRowBcast15>(a));
  b = B::f(b, dpp<kRowBcast15>(b));
  c = C::f(c, dpp<kRowBcast15>(c));
  a = A::f(a, dpp<kRowBcast31>(a));
  b = B::f(b, dpp<kRowBcast31>(b));
  c = C::f(c, dpp<kRowBcast31>(c));
  a = lane63(a);
  b = lane63(b);
  c = lane63(c);
}

// Output rows assembled in LDS, for emissions over several slots: put()
// writes a survivor's value bits and column at its rank in the wave's area
// (value at entry e, column at entry KE + e, so one address serves both),
// and flush() stores each array of the row with one coalesced store per 64
// entries. Straight to memory, an emission over several slots writes each
// 128-byte output line in parts, one store per slot. Lanes not selected
// all write one spare entry, k + 63 (as in count_and_stage); entries past
// k are never stored. Ranks past k arise only when more than k elements tie
// at the row maximum: with CLAMP (the area does not hold a whole row) they
// are clamped to the spare entry.
template <int KE, bool CLAMP>
struct StagedOut {
  uint32_t* area;
  uint32_t spare;

  __device__ __forceinline__ StagedOut(uint32_t* a, int k, int /*lane*/)
      : area(a), spare(static_cast<uint32_t>(k + kWave - 1)) {}

  __device__ __forceinline__ void put(uint64_t msk, uint32_t rank, float x,
                                      int col) const {
    uint32_t pos = lane_select(msk, rank, spare);
    if constexpr (CLAMP) pos = min(pos, spare);
    area[pos] = __float_as_uint(x);
    area[KE + pos] = static_cast<uint32_t>(col);
  }

  // Store entries 0 .. k-1 through `out` (whose buffer bounds drop the
  // positions past k of the last pass).
  template <typename Out>
  __device__ __forceinline__ void flush(const Out& out, int k, int lane) const {
    // LDS operations of one wave complete in issue order; the barriers only
    // keep the compiler from moving the reads across the writes.
    __builtin_amdgcn_wave_barrier();
#pragma unroll 1
    for (int base = 0; base < k; base += kWave) {
      const uint32_t i = static_cast<uint32_t>(base + lane);
      out.store_entry(i, area[i], area[KE + i]);
    }
    __builtin_amdgcn_wave_barrier();
  }
};

// The bracket (uniform values), #{x >= lo} (kept only while the search may
// still compact), #{x >= hi} once a count has set hi (else -1), and the
// number of counts made.
struct CappedState {
  float lo, hi;
  int clo;
  int chi;
  uint32_t steps;
};

// One specified step on the elements in `w` (the row, or the candidates):
// false once the search has stopped. A count of exactly k sets lo = hi = mid,
// after which the split test (or the width test) ends the search at the next
// step, exactly as the specified immediate stop would (nothing changes in
// between). With eps = 0 the width test is implied by the split test and is
// left out. TRACK: also keep #{x >= lo}.
template <bool EPS0, bool TRACK, int S, bool CHI = true>
__device__ __forceinline__ bool capped_step(const float (&w)[S], CappedState& b,
                                            const SelectArgs& a) {
  // max_iter < 0 (no cap) compares as the largest unsigned count.
  if (!(b.steps < static_cast<uint32_t>(a.max_iter))) return false;
  // Conditions on the uniform floats are taken as lane masks (all lanes
  // agree), which the scalar unit tests directly.
  if constexpr (!EPS0) {
    if (ballot(b.hi - b.lo > a.eps) == 0) return false;
  }
  const float mid = 0.5f * b.lo + 0.5f * b.hi;
  if ((ballot(b.lo < mid) & ballot(mid < b.hi)) == 0) return false;
  const int c = count_ge(w, mid);
  ++b.steps;
  if constexpr (TRACK) b.clo = c >= a.k ? c : b.clo;
  if constexpr (CHI) b.chi = c <= a.k ? c : b.chi;
  b.lo = c >= a.k ? mid : b.lo;
  b.hi = c <= a.k ? mid : b.hi;
  return true;
}

// Steps until the search stops. Over the candidates (S <= 2 slots) the
// steps leave #{x >= hi} to a count at the end, which costs less than
// keeping it at every step.
template <bool EPS0, int S>
__device__ __forceinline__ void capped_run(const float (&w)[S], CappedState& b,
                                           const SelectArgs& a) {
  constexpr bool kChi = S > 2;
#pragma unroll 1
  while (capped_step<EPS0, false, S, kChi>(w, b, a)) {
  }
  if constexpr (!kChi) b.chi = -1;
}

// Steps until the search stops (false) or #{x >= lo} fits `window` (true).
template <bool EPS0, int S>
__device__ __forceinline__ bool capped_run_until(const float (&w)[S],
                                                 CappedState& b,
                                                 const SelectArgs& a, int window) {
#pragma unroll 1
  for (;;) {
    if (b.clo <= window) return true;
    if (!capped_step<EPS0, true>(w, b, a)) return false;
  }
}

// The tie fill over `w`, with #{x >= hi} taken from the search when a count
// set hi (counted here only when hi is still the row maximum).
// Whether a capped kernel has an LDS area to assemble output rows in: the
// candidate staging area, or for rows of at most 512 columns without
// candidates an area of a whole row (a few KB per wave).
template <int Q, int QC>
constexpr bool capped_staged_out() {
  return QC > 0 || (Q > 1 && Q <= 8);
}

// Emissions over several slots go through `staged` (an LDS area holding the
// row's k entries) where the kernel has one, else straight to `out`.
template <bool STAGE, int S, typename Out, typename Staged, typename ColFn>
__device__ __forceinline__ void capped_emit(const float (&w)[S], ColFn col,
                                            const CappedState& b, int k,
                                            const Out& out, const Staged& staged,
                                            int lane) {
  const int nA = b.chi >= 0 ? b.chi : count_ge(w, b.hi);
  if constexpr (S == 1 || !STAGE) {
    emit_fill(w, col, b.lo, b.hi, k, nA, out);
  } else {
    emit_fill(w, col, b.lo, b.hi, k, nA, staged);
    staged.flush(out, k, lane);
  }
}

// The tie fill when lo lies below the staging threshold t0 but hi does not
// (hi is the row maximum or a midpoint whose count was at most k, both
// >= t0): A = {x >= hi} lies wholly among the candidates, and only the
// first k - nA elements of B = {lo <= x < hi} (by column) survive, which
// usually sit in the row's first slot or two. So the row is scanned slot by
// slot only until B's quota is met (the full second pass on those columns),
// and the elements of A in later columns come from the candidates, which
// are in column order. Writes exactly what emit_fill over the row would.
template <int Q, int QC, typename Out>
__device__ __forceinline__ void emit_fill_split(const float (&v)[Q],
                                                const float (&cv)[QC],
                                                const int (&ci)[QC], int lane,
                                                float lo, float hi, int k, int nA,
                                                const Out& out) {
  if (nA >= k) {
    // The first k of A, all candidates.
    emit_fill(cv, [&ci](int s) { return ci[s]; }, lo, hi, k, nA, out);
    return;
  }
  const uint32_t need = static_cast<uint32_t>(k - nA);
  uint32_t base = 0, baseB = 0;
  int end_col = kWave * Q;
#pragma unroll
  for (int s = 0; s < Q; ++s) {
    if (baseB >= need) {
      end_col = kWave * s;
      break;
    }
    const uint64_t mA = ballot(v[s] >= hi);
    const uint64_t mB = ballot(v[s] >= lo) & ~mA;
    const uint64_t keepB = ballot(rank_below(mB, baseB) < need) & mB;
    const uint64_t mS = mA | keepB;
    out.put(mS, rank_below(mS, base), v[s], s * kWave + lane);
    baseB += popc(mB);
    base += popc(mS);
  }
#pragma unroll
  for (int j = 0; j < QC; ++j) {
    const uint64_t mA = ballot(cv[j] >= hi && ci[j] >= end_col);
    out.put(mA, rank_below(mA, base), cv[j], ci[j]);
    base += popc(mA);
  }
}

// Each lane's sum of squares of a row as loaded (tail positions read as 0),
// before the wave-wide sum.
template <int Q>
__device__ __forceinline__ float lane_sum_sq(const float (&vin)[Q]) {
  float s2 = 0.0f;
#pragma unroll
  for (int s = 0; s < Q; ++s) s2 = fmaf(vin[s], vin[s], s2);
  return s2;
}

// The row's minimum (tail positions, -inf after mask_tail, left out: the
// inputs are finite) and maximum over one lane's slots.
template <int Q, bool FULL>
__device__ __forceinline__ void lane_min_max(const float (&v)[Q], float& mn, float& mx) {
  mn = kInf;
  mx = -kInf;
#pragma unroll
  for (int s = 0; s < Q; ++s) {
    mn = fminf(mn, FULL || v[s] > -kInf ? v[s] : kInf);
    mx = fmaxf(mx, v[s]);
  }
}

// GIVEN: the caller has reduced the row's minimum and maximum (and for
// QC > 0 its sum of squares) together with those of its group's other rows
// (mn_g, mx_g, s2_g); otherwise they are computed here.
template <int Q, bool FULL, int QC, bool GIVEN, typename Out>
__device__ __forceinline__ void capped_row(const float (&vin)[Q], float mn_g,
                                           float mx_g, float s2_g,
                                           const SelectArgs& a, int lane,
                                           uint32_t* __restrict__ scratch,
                                           const Out& out) {
  const int k = a.k;
  float v[Q];
#pragma unroll
  for (int s = 0; s < Q; ++s) v[s] = vin[s];
  // Sum of squares (tail positions were read as 0).
  float s2 = 0.0f;
  if constexpr (QC > 0 && !GIVEN) s2 = lane_sum_sq(vin);
  mask_tail<Q, FULL>(a.m, lane, v);
  float mn, mx;
  if constexpr (!GIVEN) lane_min_max<Q, FULL>(v, mn, mx);
  const bool eps0 = a.eps == 0.0f;
  auto row_col = [lane](int s) { return s * kWave + lane; };
  // The area the output rows are assembled in: the candidate staging area
  // (free again once the candidates are in registers), which holds k + 64
  // entries per array whenever a window is built, or for QC == 0 an area of
  // a whole row (see rows_in_registers).
  constexpr bool kStage = capped_staged_out<Q, QC>();
  constexpr int kKE = QC > 0 ? stage_entries<Q, QC>() : kWave * Q + kWave;
  const StagedOut<kKE, (!stage_whole_row<Q>() && QC > 0)> staged(scratch, k, lane);
  if constexpr (QC == 0) {
    if constexpr (GIVEN) {
      mn = mn_g;
      mx = mx_g;
    } else {
      wave_reduce2<OpMin, OpMax>(mn, mx);
    }
    CappedState b{mn, mx, a.m, -1, 0u};
    if (eps0) capped_run<true>(v, b, a); else capped_run<false>(v, b, a);
    capped_emit<kStage>(v, row_col, b, k, out, staged, lane);
  } else {
    constexpr int kW = kWave * QC;
    float cv[QC];
    int ci[QC];
    auto cand_col = [&ci](int s) { return ci[s]; };
    {
      if constexpr (GIVEN) {
        mn = mn_g;
        mx = mx_g;
        s2 = s2_g;
      } else {
        wave_reduce3<OpMin, OpMax, OpAdd>(mn, mx, s2);
      }
      CappedState b{mn, mx, a.m, -1, 0u};
      // As in exact_row: r = sqrt(sum of squares), clamped so that the
      // threshold stays finite; the model only chooses where to stage.
      const float r = fminf(__builtin_amdgcn_sqrtf(s2), 1.0e35f);
      const float t0 = r * a.z_first;
      const int c0 = count_and_stage<Q, QC>(v, t0, lane, scratch);
      if (c0 > k && c0 <= kW) {
        read_candidates<Q, QC>(scratch, c0, lane, cv, ci);
        if (eps0) capped_run<true>(cv, b, a); else capped_run<false>(cv, b, a);
        // #{x >= hi} over the candidates is the row's: hi is the row maximum
        // or a midpoint whose count was at most k, both >= t0.
        if (ballot(b.lo >= t0) != 0) {
          capped_emit<kStage>(cv, cand_col, b, k, out, staged, lane);
        } else {
          const int nA = b.chi >= 0 ? b.chi : count_ge(cv, b.hi);
          emit_fill_split(v, cv, ci, lane, b.lo, b.hi, k, nA, staged);
          staged.flush(out, k, lane);
        }
        return;
      }
      // The first count missed the window: the row from the start.
      const bool fits = eps0 ? capped_run_until<true>(v, b, a, kW)
                             : capped_run_until<false>(v, b, a, kW);
      if (fits) {
        count_and_stage<Q, QC>(v, b.lo, lane, scratch);
        read_candidates<Q, QC>(scratch, b.clo, lane, cv, ci);
        if (eps0) capped_run<true>(cv, b, a); else capped_run<false>(cv, b, a);
        capped_emit<kStage>(cv, cand_col, b, k, out, staged, lane);
      } else {
        capped_emit<kStage>(v, row_col, b, k, out, staged, lane);
      }
    }
  }
}

// Full-row search when the first count missed the candidate window: Newton
// steps on the whole row (compacting as soon as a count lands in (k, W]),
// then order-key bisection on the whole row, preceded by snaps for some row
// lengths. The snaps matter for rows with many equal values (each settles
// one distinct value); on 16,384 rows with about 30 distinct values: 512
// columns, k = 256 (no candidate window fits) 50.1 -> 18.4 us; 4,096
// columns, k = 64, 182 -> 107 us; 8,192 columns, k = 64, 374 -> 196 us. At
// 16 and 32 slots they cost occupancy (VGPRs 65 -> 79 and 86 -> 113) for
// rows that almost always land in the candidate window, so those keep key
// bisection alone.
template <int Q>
constexpr bool full_row_snaps() {
  return Q <= 8 || Q >= 64;
}

template <int Q, int QC, typename Out>
__device__ __forceinline__ void exact_row_search(const float (&v)[Q], int k,
                                              int lane, float t, int c,
                                              float h,
                                              uint32_t* __restrict__ scratch,
                                              const Out& out) {
  constexpr int kW = kWave * QC;
  const int target2 = QC > 0 ? k + kW : 2 * k + 1;
  const float h2 = 2.0f * h;
  const float shift = -static_cast<float>(target2) * h;
  auto col = [lane](int s) { return s * kWave + lane; };
  float lo = -kInf, hi = kInf;
  int clo = kWave * Q, chi = 0;  // #{x >= lo} (padding included), #{x >= hi}
#pragma unroll 1
  for (int it = 1;; ++it) {
    const bool up = c > k;
    lo = up ? t : lo;
    clo = up ? c : clo;
    hi = up ? hi : t;
    chi = up ? chi : c;
    if (it == kRowSteps) break;
    t = fmaf(static_cast<float>(c), h2, t + shift);
    c = count_ge(v, t);
    if (c == k) {
      emit_ge(v, col, t, out);
      return;
    }
    if constexpr (QC > 0) {
      if (c > k && c <= kW) {
        count_and_stage<Q, QC>(v, t, lane, scratch);
        float cv[QC];
        int ci[QC];
        read_candidates<Q, QC>(scratch, c, lane, cv, ci);
        exact_candidates<QC>(cv, ci, k, t, c, h, out);
        return;
      }
    }
  }
  if constexpr (full_row_snaps<Q>())
    settle_candidates<Q>(v, col, k, lo, clo, hi, chi, out);
  else
    finish_by_keys(v, col, k, lo, hi, chi, out);
}

// s2: the row's sum of squares (wave_sum of lane_sum_sq), the scale of the
// row for the model behind the thresholds (the model assumes rows centred
// near zero; the Newton steps correct the first threshold when they are
// not). With S2_GIVEN the caller has reduced the sums of a group's rows
// together; otherwise it is computed here.
template <int Q, bool FULL, int QC, bool S2_GIVEN, typename Out>
__device__ __forceinline__ void exact_row(const float (&vin)[Q], float s2,
                                          const SelectArgs& a, int lane,
                                          uint32_t* __restrict__ scratch,
                                          const Out& out) {
  const int k = a.k;
  if constexpr (!S2_GIVEN) s2 = wave_sum(lane_sum_sq(vin));
  float v[Q];
#pragma unroll
  for (int s = 0; s < Q; ++s) v[s] = vin[s];
  mask_tail<Q, FULL>(a.m, lane, v);
  // r = sqrt(sum of squares) = rms * sqrt(m); the host folded 1/sqrt(m) into
  // the model constants. Raw hardware square root: the model only steers
  // the search. Clamping r keeps every threshold finite: the first is at
  // most ~4r, each Newton step moves by at most (2m + 1) h <= ~50r (h is at
  // most 1.25r), and there are at most 8 steps, so |t| < 1e38. Rows whose
  // squares overflow (~1.8e19) get the clamped scale; the search then
  // relies on its bounded fallbacks.
  const float r = fminf(__builtin_amdgcn_sqrtf(s2), 1.0e35f);
  const float h = r * a.half_step;
  const float t = r * a.z_first;
  int c;
  if constexpr (QC > 0) {
    c = count_and_stage<Q, QC>(v, t, lane, scratch);
    // c in (k, W], as one unsigned compare.
    if (static_cast<uint32_t>(c - k - 1) < static_cast<uint32_t>(kWave * QC - k)) {
      float cv[QC];
      int ci[QC];
      read_candidates<Q, QC>(scratch, c, lane, cv, ci);
      exact_candidates<QC>(cv, ci, k, t, c, h, out);
      return;
    }
  } else {
    c = count_ge(v, t);
  }
  if (c == k) {
    emit_ge(v, [lane](int s) { return s * kWave + lane; }, t, out);
    return;
  }
  // The first count missed the window: the row is not centred near zero, or
  // not shaped like a normal sample. One retry with the row's own mean and
  // standard deviation (shifted, one-sided or uniform rows then land in the
  // window; measured at 262,144 x 256: N(0,1) + 1000 300 -> 62 us, -(U(0,1)
  // + 5) 260 -> 80 us, U(0,1) 187 -> 79 us). Computing them for every row
  // instead cost 5% on N(0,1) rows, where 99.5% of first counts land.
  // The model only steers: sums that overflow or cancel to NaN are
  // replaced by values that keep every threshold finite (|mean| <= 1e37,
  // sd <= 1e33; a step then moves by at most (2m + 1) h <= ~1.5e36 and
  // there are at most 9 of them, so |t| < 3e37).
  {
    auto finite_or = [](float x, float y) {
      return (__float_as_uint(x) & 0x7f800000u) != 0x7f800000u ? x : y;
    };
    float s1 = 0.0f;
#pragma unroll
    for (int s = 0; s < Q; ++s) s1 += FULL ? v[s] : finite_or(v[s], 0.0f);  // tail: -inf
    s1 = wave_sum(s1);
    const float mean = fminf(fmaxf(finite_or(s1 * a.inv_m, 0.0f), -1.0e37f), 1.0e37f);
    const float var = finite_or(fmaf(-mean, mean, s2 * a.inv_m), 1.0e38f);
    const float sd = fminf(__builtin_amdgcn_sqrtf(fmaxf(var, 0.0f)), 1.0e33f);
    const float h1 = sd * a.half_step_c;
    const float t1 = fmaf(sd, a.z_first_c, mean);
    // Rows of 8,192 columns: a retry threshold that moves the expected
    // count by less than a quarter of the candidate window ((W - k) / 4
    // elements; a step of h moves it by one half, and the smaller of the two
    // models' steps is the scale) would count about the same elements again,
    // as happens on rows centred near zero with many equal values whose
    // first count jumped over the window; those carry on from the first
    // count. On shorter rows the retry pays even then and always runs.
    bool near = false;
    if constexpr (QC > 0 && Q >= 128)
      near = 2.0f * fabsf(t1 - t) < static_cast<float>(kWave * QC - k) * fminf(h, h1);
    if (!near) {
      int c1;
      if constexpr (QC > 0) {
        c1 = count_and_stage<Q, QC>(v, t1, lane, scratch);
        if (static_cast<uint32_t>(c1 - k - 1) < static_cast<uint32_t>(kWave * QC - k)) {
          float cv[QC];
          int ci[QC];
          read_candidates<Q, QC>(scratch, c1, lane, cv, ci);
          exact_candidates<QC>(cv, ci, k, t1, c1, h1, out);
          return;
        }
      } else {
        c1 = count_ge(v, t1);
      }
      if (c1 == k) {
        emit_ge(v, [lane](int s) { return s * kWave + lane; }, t1, out);
        return;
      }
      // Carry on from whichever count came nearer to the window's middle.
      const int mid2 = QC > 0 ? k + kWave * QC : 2 * k + 1;  // twice the middle
      const bool second = abs(2 * c1 - mid2) < abs(2 * c - mid2);
      if (second) {
        exact_row_search<Q, QC>(v, k, lane, t1, c1, h1, scratch, out);
        return;
      }
    }
  }
  exact_row_search<Q, QC>(v, k, lane, t, c, h, scratch, out);
}

// ---------------------------------------------------------------------------
// The kernel: each wave takes groups of rows, one row at a time.
// ---------------------------------------------------------------------------
// GIVEN: the row's reductions (s2; for the capped search also mn, mx) were
// taken with those of its group's other rows.
template <int Q, bool FULL, Mode MODE, int QC, bool GIVEN, typename Out>
__device__ __forceinline__ void process_row(const float (&v)[Q], float mn, float mx,
                                            float s2, const SelectArgs& a, int lane,
                                            uint32_t* __restrict__ scratch,
                                            const Out& out) {
  if constexpr (MODE != Mode::kCapped)
    exact_row<Q, FULL, QC, GIVEN>(v, s2, a, lane, scratch, out);
  else
    capped_row<Q, FULL, QC, GIVEN>(v, mn, mx, s2, a, lane, scratch, out);
}

// Rows each wave keeps in flight (rows_in_flight in rtopk_internal.h): a
// group of D consecutive rows whose loads are all issued before the first
// of them is worked on.
template <int Q, Mode MODE>
constexpr int prefetch_depth() {
  return rows_in_flight(Q, MODE == Mode::kMaxk);
}

// Row order. Wave w of S works through groups of D consecutive rows:
// group g is rows (g*S + w)*D ... (g*S + w)*D + D - 1, so at any moment all
// waves together read one contiguous stretch of the matrix (HBM streams
// fastest that way). For short rows the host launches enough waves for one
// group each and the group loop runs once; long rows (D = 1) get a
// persistent grid.
//
// A group's loads are issued together, before any of its stores: loads and
// stores of a wave complete in issue order on one counter, so waiting for a
// row never waits for the stores of the rows before it. Rows past the end
// of the matrix re-read the last row (the loads stay unconditional and the
// compiler's wait counts exact) and are not processed.
template <int Q, bool FULL, Mode MODE, int QC, typename IdxT>
__global__ __launch_bounds__(kWave * row_waves(Q)) void rows_in_registers(SelectArgs a) {
  // Per wave: the LDS staging area of the exact search, (value, column)
  // pairs (see stage_entries).
  // Capped kernels without candidates: an area to assemble output rows in
  // (see StagedOut), k + 64 <= 64*Q + 64 entries per array.
  constexpr int kScratch =
      QC > 0 ? 2 * stage_entries<Q, QC>()
      : MODE == Mode::kCapped && capped_staged_out<Q, QC>() ? 2 * (kWave * Q + kWave)
                                                             : 1;
  constexpr int D = prefetch_depth<Q, MODE>();
  constexpr int kRowWaves = row_waves(Q);
  // MaxK forward: the wave's LDS copy of the dense row (64*Q words) and one
  // spare word per lane.
  constexpr bool kDense = MODE == Mode::kMaxk;
  constexpr int kDenseWords = kDense ? kWave * (Q + 1) : 1;
  constexpr bool kBuckets = MODE == Mode::kBucket;
  __shared__ uint32_t scratch_all[kRowWaves][kScratch];
  __shared__ uint32_t dense_all[kRowWaves][kDenseWords];
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  const int wave_in_block =
      __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  uint32_t* scratch = scratch_all[wave_in_block];
  uint32_t* dense = dense_all[wave_in_block];
  const uint32_t spare = static_cast<uint32_t>(kWave * Q + lane);
  const int64_t waves = static_cast<int64_t>(gridDim.x) * kRowWaves;
  const int64_t w = static_cast<int64_t>(blockIdx.x) * kRowWaves + wave_in_block;
  const int64_t stride = waves * D;
#pragma unroll 1
  for (int64_t r = w * D; r < a.n; r += stride) {
    const int rows = a.n - r < D ? static_cast<int>(a.n - r) : D;
    const float* xg = a.x + r * a.m;
    float buf[D][Q];
#pragma unroll
    for (int d = 0; d < D; ++d)
      load_row<Q, FULL>(xg + min(d, rows - 1) * a.m, a.m, lane, buf[d]);
    // Keep the group's loads here: without a memory barrier right after
    // them, code generation sinks the loads of the later rows past the
    // first row's search loop (the capped search), so that only one row is
    // in flight while it waits. No wait is implied.
    asm volatile("" ::: "memory");
    // The group's row reductions taken together (the exact search's sums
    // of squares; the capped search's minima, maxima and sums of squares):
    // one chain of dependent DPP steps instead of one per row (262,144 x
    // 256, 4 rows per group: exact 56.0 -> 53.9 us, capped with 2 steps
    // 59.6 -> 57.3 us), and with the lane swaps of wave_reduce_groups,
    // half the instructions of separate reductions (capped with 2 steps
    // 56.9 -> 55.0 us, 4 steps 59.3 -> 57.2 us). Groups of two rows (512 to
    // 1,024 columns) keep them inside the search (0.6% faster at 1,024
    // columns).
    constexpr bool kGiven = D >= 4;
    float s2g[D], mng[D], mxg[D];
    if constexpr (kGiven) {
#pragma unroll
      for (int d = 0; d < D; ++d) s2g[d] = lane_sum_sq(buf[d]);
      if constexpr (MODE == Mode::kCapped) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
          float w[Q];
#pragma unroll
          for (int s = 0; s < Q; ++s) w[s] = buf[d][s];
          mask_tail<Q, FULL>(a.m, lane, w);
          lane_min_max<Q, FULL>(w, mng[d], mxg[d]);
        }
        // Without candidates the capped search needs no sum of squares.
        if constexpr (QC > 0)
          wave_minmaxsum_n(mng, mxg, s2g);
        else
          wave_minmax_n(mng, mxg);
      } else {
        wave_sum_n(s2g);
      }
    }
    float* og = a.out_val + r * a.k;
    IdxT* ig = static_cast<IdxT*>(a.out_idx) + r * a.k;
    float* yg = kDense ? a.dense + r * a.m : nullptr;
    // kBucket: bucket index of row r within its input row; rows of a group
    // are consecutive, so it then advances with a wrap.
    int bucket = 0;
    if constexpr (kBuckets) {
      bucket = r < 0x100000000LL
                   ? static_cast<int>(static_cast<uint32_t>(r) %
                                      static_cast<uint32_t>(a.buckets))
                   : static_cast<int>(r % a.buckets);
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      if (d >= rows) break;
      if constexpr (kDense) {
#pragma unroll
        for (int s = 0; s < Q; ++s) dense[s * kWave + lane] = 0u;
        // LDS operations of one wave complete in issue order; the barriers
        // keep the compiler from moving them across each other.
        __builtin_amdgcn_wave_barrier();
      }
      process_row<Q, FULL, MODE, QC, kGiven>(
          buf[d], kGiven && MODE == Mode::kCapped ? mng[d] : 0.0f,
          kGiven && MODE == Mode::kCapped ? mxg[d] : 0.0f, kGiven ? s2g[d] : 0.0f, a, lane,
          scratch,
          OutRow<IdxT, MODE>(og + d * a.k, ig + d * a.k, a.k, dense, spare,
                             bucket * a.m));
      if constexpr (kBuckets) bucket = bucket + 1 == a.buckets ? 0 : bucket + 1;
      if constexpr (kDense) {
        __builtin_amdgcn_wave_barrier();
        // The dense row, stores past its end dropped.
        const __amdgpu_buffer_rsrc_t ry = __builtin_amdgcn_make_buffer_rsrc(
            yg + d * a.m, 0, a.m * 4, kRsrcWord3);
#pragma unroll
        for (int s = 0; s < Q; ++s)
          __builtin_amdgcn_raw_buffer_store_b32(dense[s * kWave + lane], ry,
                                                (s * kWave + lane) * 4, 0, kStoreNT);
        __builtin_amdgcn_wave_barrier();
      }
    }
  }
}

// Candidate slot counts QC the exact kernels are built with for Q slots:
// 0 (no compaction) and the powers of two up to Q/2.
constexpr bool exact_qc_built(int q, int qc) {
  return qc == 0 || ((qc == 1 || qc == 2 || qc == 4 || qc == 8) && 2 * qc <= q);
}

template <int Q, bool FULL, Mode MODE, typename IdxT>
RowsKernel exact_kernel(int qc) {
  switch (qc) {
    case 1:
      if constexpr (exact_qc_built(Q, 1))
        return rows_in_registers<Q, FULL, MODE, 1, IdxT>;
      break;
    case 2:
      if constexpr (exact_qc_built(Q, 2))
        return rows_in_registers<Q, FULL, MODE, 2, IdxT>;
      break;
    case 4:
      if constexpr (exact_qc_built(Q, 4))
        return rows_in_registers<Q, FULL, MODE, 4, IdxT>;
      break;
    case 8:
      if constexpr (exact_qc_built(Q, 8))
        return rows_in_registers<Q, FULL, MODE, 8, IdxT>;
      break;
    default:
      break;
  }
  return rows_in_registers<Q, FULL, MODE, 0, IdxT>;
}

template <int Q, bool FULL, typename IdxT>
RowsKernel any_kernel(Mode mode, int qc) {
  if (mode == Mode::kExact) return exact_kernel<Q, FULL, Mode::kExact, IdxT>(qc);
  if (mode == Mode::kMaxk) {
    if constexpr (maxk_fused(Q)) return exact_kernel<Q, FULL, Mode::kMaxk, IdxT>(qc);
    return nullptr;
  }
  if (mode == Mode::kBucket) {
    if constexpr (bucket_supported(Q)) return exact_kernel<Q, FULL, Mode::kBucket, IdxT>(qc);
    return nullptr;
  }
  return exact_kernel<Q, FULL, Mode::kCapped, IdxT>(qc);
}

}  // namespace rows_detail

// The row kernel for Q slots per lane (row length up to 64*Q), one of the
// buckets listed in rtopk_internal.h. full: the row length is exactly 64*Q
// (only distinguished for Q <= 4). qc: candidate slots for the exact search
// (see candidate_slots). Returns nullptr for one-byte indices with Q > 4,
// and for Mode::kMaxk / kBucket with rows too long for those kernels.
template <int Q>
RowsKernel rows_kernel(bool full, Mode mode, bool u8_index, int qc) {
  using rows_detail::any_kernel;
  if (u8_index) {
    if constexpr (Q <= 4) {
      return full ? any_kernel<Q, true, uint8_t>(mode, qc)
                  : any_kernel<Q, false, uint8_t>(mode, qc);
    } else {
      return nullptr;
    }
  }
  if constexpr (Q <= 4) {
    if (full) return any_kernel<Q, true, int32_t>(mode, qc);
  }
  return any_kernel<Q, false, int32_t>(mode, qc);
}

}  // namespace rtopk
