#pragma once

// Row-wise top-k for long rows: one row per group of four waves (one block).
//
// Method: the exact search and the capped search of rtopk_rows.hpp (RTop-K
// summary page, "Approach": a threshold search over the row's values, then
// the k survivors in column order), with the row spread over the four waves
// of a block.
//
// Why: a row of 8,192 floats held by one wave takes 128 registers per lane,
// so each SIMD runs one such wave and a CU has four rows in flight, each
// loaded and then searched with nothing of its own overlapping. Held by four
// waves, a row takes 32 registers per lane and is searched by four waves at
// once; more rows fit on a CU, and each spends a quarter of the time in its
// search.
//
// Layout: wave g of the block holds columns [64*Q*g, 64*Q*(g+1)) of the row,
// lane l and slot s holding column 64*Q*g + 64*s + l, so the columns of the
// row are in (wave, slot, lane) order and each wave's load is one contiguous
// stretch.
//
// Everything the search decides on is a row-level value: each count (and
// sum, minimum, maximum) is taken per wave and combined through LDS, with
// one barrier per combination. Every wave therefore computes the same
// thresholds and takes the same branches, and reaches the same barriers.
// Candidates (elements above a threshold, when their count fits the window)
// are written by each wave to an LDS area of its own and read back as one
// list in column order. The exact search on them needs no exchange and
// runs in wave 0 alone, which assembles its output row in an LDS output
// area and stores it coalesced; the capped search runs its steps in every
// wave alike (the branch after them may need the whole group) and wave 0
// stores what it emits from the candidates directly (assembling those rows
// too measured 4-10% slower at 2 steps). Emissions over the whole row write
// each wave's own columns at ranks offset by the survivors of the waves
// before it.

#include "rtopk_rows.hpp"

namespace rtopk {
namespace group_detail {

using namespace rows_detail;

// Waves per row.
constexpr int kG = kWavesPerRowGroup;

// The row group's LDS exchange and this wave's place in it.
struct Group {
  int g;          // wave index in the group (uniform)
  int lane;
  uint32_t* xch;  // [2][kG][2] words, then 64 spare words
  uint32_t parity;
  int part[kG];   // per-wave counts of the last row_count

  // Publish two words per wave and read every wave's (a[i], b[i]). The two
  // halves of the area alternate, so one barrier per exchange suffices: a
  // wave writes a half again only after the next exchange's barrier, which
  // every wave reaches after its reads of this one.
  __device__ __forceinline__ void exchange2(uint32_t va, uint32_t vb,
                                            uint32_t (&a)[kG], uint32_t (&b)[kG]) {
    uint32_t* half = xch + parity * (2 * kG);
    // Lane 0 writes the wave's slot, the other lanes a spare word of their
    // own (no exec-mask change, no two lanes on one word).
    const uint32_t spare = 4 * kG + static_cast<uint32_t>(lane);
    uint32_t* dst = lane == 0 ? half + 2 * g : xch + spare;
    dst[0] = va;
    dst[lane == 0 ? 1 : kWave] = vb;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kG; ++i) {
      a[i] = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(half[2 * i])));
      b[i] = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(half[2 * i + 1])));
    }
    parity ^= 1u;
  }

  __device__ __forceinline__ void exchange1(uint32_t v, uint32_t (&a)[kG]) {
    uint32_t b[kG];
    exchange2(v, 0u, a, b);
  }

  // Sum over the waves of the part of the last row_count before this wave.
  __device__ __forceinline__ int prefix() const {
    int p = 0;
#pragma unroll
    for (int i = 0; i < kG; ++i) p += i < g ? part[i] : 0;
    return p;
  }
};

// #{x >= t} over the row (and the per-wave parts, for emit_ge).
template <int Q>
__device__ __forceinline__ int row_count(Group& G, const float (&v)[Q], float t) {
  uint32_t all[kG];
  G.exchange1(static_cast<uint32_t>(count_ge(v, t)), all);
  int c = 0;
#pragma unroll
  for (int i = 0; i < kG; ++i) {
    G.part[i] = static_cast<int>(all[i]);
    c += G.part[i];
  }
  return c;
}

// Row-wide reductions, combined in wave order (the same value in every wave).
__device__ __forceinline__ float row_sum(Group& G, float x) {
  uint32_t all[kG];
  G.exchange1(__float_as_uint(wave_sum(x)), all);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kG; ++i) s += __uint_as_float(all[i]);
  return s;
}

// Sum over the waves of values already reduced within each wave.
__device__ __forceinline__ float row_sum_of_waves(Group& G, float wave_total) {
  uint32_t all[kG];
  G.exchange1(__float_as_uint(wave_total), all);
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kG; ++i) s += __uint_as_float(all[i]);
  return s;
}

__device__ __forceinline__ float row_max(Group& G, float x) {
  uint32_t all[kG];
  G.exchange1(__float_as_uint(wave_max(x)), all);
  float s = -kInf;
#pragma unroll
  for (int i = 0; i < kG; ++i) s = fmaxf(s, __uint_as_float(all[i]));
  return s;
}

__device__ __forceinline__ float row_min(Group& G, float x) {
  uint32_t all[kG];
  G.exchange1(__float_as_uint(wave_min(x)), all);
  float s = kInf;
#pragma unroll
  for (int i = 0; i < kG; ++i) s = fminf(s, __uint_as_float(all[i]));
  return s;
}

// Every element >= t, in column order; the last row_count was at t (and
// found exactly k).
template <int Q, typename Out, typename ColFn>
__device__ __forceinline__ void row_emit_ge(const Group& G, const float (&v)[Q],
                                            ColFn col, float t, const Out& out) {
  // Recompute the compares rather than let the compiler keep the lane masks
  // of the count that found t alive across the exchange (one scalar pair per
  // slot, spilled).
  asm volatile("" : "+v"(t));
  uint32_t base = static_cast<uint32_t>(G.prefix());
#pragma unroll
  for (int s = 0; s < Q; ++s) {
    const uint64_t msk = ballot(v[s] >= t);
    out.put(msk, rank_below(msk, base), v[s], col(s));
    base += popc(msk);
  }
}

// The second pass over the row (emit_fill's rule: the first k by column of
// A = {x >= hi}, then of B = {lo <= x < hi}; #{x >= lo} >= k). Each wave
// first counts its A and B, the counts are exchanged, and each wave then
// emits its columns at ranks after those of the waves before it.
template <int Q, typename Out, typename ColFn>
__device__ __forceinline__ void row_emit_fill(Group& G, const float (&v)[Q],
                                              ColFn col, float lo, float hi, int k,
                                              const Out& out) {
  int na = 0, nb = 0;
#pragma unroll
  for (int s = 0; s < Q; ++s) {
    const uint64_t mA = ballot(v[s] >= hi);
    na += popc(mA);
    nb += popc(ballot(v[s] >= lo) & ~mA);
  }
  uint32_t as[kG], bs[kG];
  G.exchange2(static_cast<uint32_t>(na), static_cast<uint32_t>(nb), as, bs);
  // The emission recomputes its compares (see row_emit_ge).
  asm volatile("" : "+v"(lo));
  asm volatile("" : "+v"(hi));
  int nA = 0, preA = 0, preB = 0;
#pragma unroll
  for (int i = 0; i < kG; ++i) {
    nA += static_cast<int>(as[i]);
    preA += i < G.g ? static_cast<int>(as[i]) : 0;
    preB += i < G.g ? static_cast<int>(bs[i]) : 0;
  }
  if (nA >= k) {
    // The first k of A: ranks past k are dropped by the output bounds.
    uint32_t base = static_cast<uint32_t>(preA);
#pragma unroll
    for (int s = 0; s < Q; ++s) {
      const uint64_t mA = ballot(v[s] >= hi);
      out.put(mA, rank_below(mA, base), v[s], col(s));
      base += popc(mA);
    }
    return;
  }
  const uint32_t need = static_cast<uint32_t>(k - nA);
  // The waves before this one keep min(preB, need) elements of B.
  uint32_t base = static_cast<uint32_t>(preA) + min(static_cast<uint32_t>(preB), need);
  uint32_t baseB = static_cast<uint32_t>(preB);
#pragma unroll
  for (int s = 0; s < Q; ++s) {
    const uint64_t mA = ballot(v[s] >= hi);
    const uint64_t mB = ballot(v[s] >= lo) & ~mA;
    const uint64_t keepB = ballot(rank_below(mB, baseB) < need) & mB;
    const uint64_t mS = mA | keepB;
    out.put(mS, rank_below(mS, base), v[s], col(s));
    baseB += popc(mB);
    base += popc(mS);
  }
}

// Order-key bisection over the row (finish_by_keys, row-wide).
template <int Q, typename Out, typename ColFn>
__device__ __forceinline__ void row_finish_by_keys(Group& G, const float (&v)[Q],
                                                   ColFn col, int k, float lo,
                                                   float hi, const Out& out) {
  int32_t klo = order_key(lo);
  int32_t khi = order_key(hi);
#pragma unroll 1
  for (;;) {
    const uint32_t width = static_cast<uint32_t>(khi) - static_cast<uint32_t>(klo);
    if (width <= 1u) break;
    const int32_t kmid =
        static_cast<int32_t>(static_cast<uint32_t>(klo) + (width >> 1));
    const float t = key_value(kmid);
    const int c = row_count(G, v, t);
    if (c == k) {
      row_emit_ge(G, v, col, t, out);
      return;
    }
    const bool up = c > k;
    klo = up ? kmid : klo;
    khi = up ? khi : kmid;
  }
  row_emit_fill(G, v, col, key_value(klo), key_value(khi), k, out);
}

// Snaps over the row (settle_candidates, row-wide), then key bisection.
template <int Q, typename Out, typename ColFn>
__device__ __forceinline__ void row_settle(Group& G, const float (&v)[Q],
                                           ColFn col, int k, float lo, int clo,
                                           float hi, int chi, const Out& out) {
#pragma unroll 1
  for (int it = 0; it < kCandSnaps; ++it) {
    const int need = k - chi;
    const int span = clo - chi;
    if (need <= span - need + 1) {
      float u = -kInf;
#pragma unroll
      for (int s = 0; s < Q; ++s) u = fmaxf(u, v[s] < hi ? v[s] : -kInf);
      u = row_max(G, u);
      const int cu = row_count(G, v, u);
      if (cu >= k) {
        row_emit_fill(G, v, col, u, hi, k, out);
        return;
      }
      hi = u;
      chi = cu;
    } else {
      float u = kInf;
#pragma unroll
      for (int s = 0; s < Q; ++s) u = fminf(u, v[s] >= lo ? v[s] : kInf);
      u = row_min(G, u);
      const float above = next_float(u);
      const int cg = row_count(G, v, above);
      if (cg <= k) {
        row_emit_fill(G, v, col, u, above, k, out);
        return;
      }
      lo = above;
      clo = cg;
    }
  }
  row_finish_by_keys(G, v, col, k, lo, hi, out);
}

// LDS candidate area of one wave: values at [0, E), columns at [E, 2E),
// E = kWave * QC + kWave (the candidates of one wave never exceed the row's
// window; ranks past it go to the spare entry).
template <int QC>
constexpr int sub_entries() {
  return kWave * QC + kWave;
}

// #{x >= t} over the row; each wave also writes its elements >= t, in column
// order, to its own candidate area (see count_and_stage: the lanes not
// writing a candidate all write the last entry).
template <int Q, int QC>
__device__ __forceinline__ int row_count_and_stage(Group& G, const float (&v)[Q],
                                                   float t, int col0,
                                                   uint32_t* __restrict__ area) {
  constexpr uint32_t kE = sub_entries<QC>();
  constexpr uint32_t spare = kWave * QC + kWave - 1;
  uint32_t base = 0;
#pragma unroll
  for (int s = 0; s < Q; ++s) {
    const uint64_t msk = ballot(v[s] >= t);
    const uint32_t e = min(lane_select(msk, rank_below(msk, base), spare), spare);
    area[e] = __float_as_uint(v[s]);
    area[kE + e] = static_cast<uint32_t>(col0 + s * kWave + G.lane);
    base += popc(msk);
  }
  uint32_t all[kG];
  G.exchange1(base, all);
  int c = 0;
#pragma unroll
  for (int i = 0; i < kG; ++i) {
    G.part[i] = static_cast<int>(all[i]);
    c += G.part[i];
  }
  return c;
}

// The row's c candidates (c <= 64*QC), in column order, into QC slots (every
// wave's writes came before the barrier of the exchange that counted them):
// entry e of the list is entry e - (count of the waves before w) of wave w's
// area, w the wave whose part of the list holds e.
template <int QC>
__device__ __forceinline__ void row_read_candidates(const Group& G,
                                                    const uint32_t* __restrict__ areas,
                                                    int c, float (&cv)[QC],
                                                    int (&ci)[QC]) {
  constexpr int kE = sub_entries<QC>();
  const int p1 = G.part[0];
  const int p2 = p1 + G.part[1];
  const int p3 = p2 + G.part[2];
#pragma unroll
  for (int j = 0; j < QC; ++j) {
    const int e = j * kWave + G.lane;
    const int w = (e >= p1) + (e >= p2) + (e >= p3);
    const int start = e >= p3 ? p3 : e >= p2 ? p2 : e >= p1 ? p1 : 0;
    const int at = w * (2 * kE) + (e - start);
    const float x = __uint_as_float(areas[at]);
    cv[j] = e < c ? x : -kInf;
    ci[j] = static_cast<int>(areas[at + kE]);
  }
}

// Entries per array of wave 0's LDS output area: k + 64 (k <= 32 QC, as
// the window holds at least 2k candidates).
template <int QC>
constexpr int out_entries() {
  return QC > 0 ? 32 * QC + kWave : 1;
}

// The exact search on the row's candidates (exact_candidates) by wave 0
// alone: it needs no exchange, so the other waves have nothing left to do
// for the row. Wave 0 assembles the output row in its LDS output area and
// stores it with coalesced stores (straight from several candidate slots,
// each output line would be written in parts).
template <int QC, typename Out>
__device__ __forceinline__ void row_candidates_exact(const Group& G,
                                                     const uint32_t* __restrict__ areas,
                                                     uint32_t* __restrict__ ostage, int c,
                                                     int k, float t, float h,
                                                     const Out& out) {
  if (G.g != 0) return;
  float cv[QC];
  int ci[QC];
  row_read_candidates<QC>(G, areas, c, cv, ci);
  const StagedOut<out_entries<QC>(), true> staged(ostage, k, G.lane);
  exact_candidates<QC>(cv, ci, k, t, c, h, staged);
  staged.flush(out, k, G.lane);
}

// Full-row Newton steps when the first count missed the window
// (exact_row_search, row-wide).
template <int Q, int QC, typename Out>
__device__ __forceinline__ void row_search(Group& G, const float (&v)[Q], int k,
                                           float t, int c, float h, int col0,
                                           uint32_t* __restrict__ areas,
                                           const Out& out, uint32_t* __restrict__ ostage) {
  constexpr int kW = kWave * QC;
  const int target2 = QC > 0 ? k + kW : 2 * k + 1;
  const float h2 = 2.0f * h;
  const float shift = -static_cast<float>(target2) * h;
  const int lane = G.lane;
  auto col = [lane, col0](int s) { return col0 + s * kWave + lane; };
  float lo = -kInf, hi = kInf;
  int clo = kG * kWave * Q, chi = 0;
#pragma unroll 1
  for (int it = 1;; ++it) {
    const bool up = c > k;
    lo = up ? t : lo;
    clo = up ? c : clo;
    hi = up ? hi : t;
    chi = up ? chi : c;
    if (it == kRowSteps) break;
    t = fmaf(static_cast<float>(c), h2, t + shift);
    if constexpr (QC > 0) {
      c = row_count_and_stage<Q, QC>(G, v, t, col0, areas + G.g * 2 * sub_entries<QC>());
    } else {
      c = row_count(G, v, t);
    }
    if (c == k) {
      row_emit_ge(G, v, col, t, out);
      return;
    }
    if constexpr (QC > 0) {
      if (c > k && c <= kW) {
        row_candidates_exact<QC>(G, areas, ostage, c, k, t, h, out);
        return;
      }
    }
  }
  row_settle(G, v, col, k, lo, clo, hi, chi, out);
}

template <int Q, bool FULL, int QC, typename Out>
__device__ __forceinline__ void row_exact(Group& G, const float (&vin)[Q],
                                          const SelectArgs& a, int m_local, int col0,
                                          uint32_t* __restrict__ areas,
                                          const Out& out, uint32_t* __restrict__ ostage) {
  const int k = a.k;
  const int lane = G.lane;
  float v[Q];
  float s2 = 0.0f;
#pragma unroll
  for (int s = 0; s < Q; ++s) {
    v[s] = vin[s];
    s2 = fmaf(vin[s], vin[s], s2);
  }
  s2 = row_sum(G, s2);
  mask_tail<Q, FULL>(m_local, lane, v);
  auto col = [lane, col0](int s) { return col0 + s * kWave + lane; };
  uint32_t* mine = areas + G.g * 2 * sub_entries<QC>();
  // The model and its bounds as in exact_row.
  const float r = fminf(__builtin_amdgcn_sqrtf(s2), 1.0e35f);
  const float h = r * a.half_step;
  const float t = r * a.z_first;
  int c;
  if constexpr (QC > 0) {
    c = row_count_and_stage<Q, QC>(G, v, t, col0, mine);
    if (static_cast<uint32_t>(c - k - 1) < static_cast<uint32_t>(kWave * QC - k)) {
      row_candidates_exact<QC>(G, areas, ostage, c, k, t, h, out);
      return;
    }
  } else {
    c = row_count(G, v, t);
  }
  if (c == k) {
    row_emit_ge(G, v, col, t, out);
    return;
  }
  // The retry with the row's mean and standard deviation (exact_row).
  {
    auto finite_or = [](float x, float y) {
      return (__float_as_uint(x) & 0x7f800000u) != 0x7f800000u ? x : y;
    };
    float s1 = 0.0f;
#pragma unroll
    for (int s = 0; s < Q; ++s) s1 += FULL ? v[s] : finite_or(v[s], 0.0f);
    s1 = row_sum(G, s1);
    const float mean = fminf(fmaxf(finite_or(s1 * a.inv_m, 0.0f), -1.0e37f), 1.0e37f);
    const float var = finite_or(fmaf(-mean, mean, s2 * a.inv_m), 1.0e38f);
    const float sd = fminf(__builtin_amdgcn_sqrtf(fmaxf(var, 0.0f)), 1.0e33f);
    const float h1 = sd * a.half_step_c;
    const float t1 = fmaf(sd, a.z_first_c, mean);
    // Rows of 8,192 columns skip a retry that would move the expected count
    // by less than a quarter of the window (as in exact_row).
    bool near = false;
    if constexpr (QC > 0 && kG * Q >= 128)
      near = 2.0f * fabsf(t1 - t) < static_cast<float>(kWave * QC - k) * fminf(h, h1);
    if (!near) {
      int c1;
      if constexpr (QC > 0) {
        c1 = row_count_and_stage<Q, QC>(G, v, t1, col0, mine);
        if (static_cast<uint32_t>(c1 - k - 1) < static_cast<uint32_t>(kWave * QC - k)) {
          row_candidates_exact<QC>(G, areas, ostage, c1, k, t1, h1, out);
          return;
        }
      } else {
        c1 = row_count(G, v, t1);
      }
      if (c1 == k) {
        row_emit_ge(G, v, col, t1, out);
        return;
      }
      const int mid2 = QC > 0 ? k + kWave * QC : 2 * k + 1;
      if (abs(2 * c1 - mid2) < abs(2 * c - mid2)) {
        row_search<Q, QC>(G, v, k, t1, c1, h1, col0, areas, out, ostage);
        return;
      }
    }
  }
  row_search<Q, QC>(G, v, k, t, c, h, col0, areas, out, ostage);
}

// The row's output assembled in LDS by all four waves (the candidate areas,
// free once every wave is past the exchange that follows its last read of
// them): put() writes a survivor's value bits at entry `rank` and its
// column at entry ke + rank; lanes not selected, and ranks past k (more
// than k elements tied at the row maximum), write the wave's spare entry,
// k + 64 g + 63 (one address for all of them, as in count_and_stage).
// flush() then stores the k entries with coalesced stores, each wave a
// quarter of them, after a barrier.
struct GroupStaged {
  uint32_t* area;
  uint32_t ke;     // entries per array: k + 64 * kG
  uint32_t spare;  // this wave's spare entry

  __device__ __forceinline__ GroupStaged(uint32_t* a, int k, int g, int /*lane*/)
      : area(a),
        ke(static_cast<uint32_t>(k + kWave * kG)),
        spare(static_cast<uint32_t>(k + kWave * g + kWave - 1)) {}

  __device__ __forceinline__ void put(uint64_t msk, uint32_t rank, float x, int col) const {
    const uint32_t pos = min(lane_select(msk, rank, spare), spare);
    area[pos] = __float_as_uint(x);
    area[ke + pos] = static_cast<uint32_t>(col);
  }

  template <typename Out>
  __device__ __forceinline__ void flush(const Group& G, const Out& out, int k) const {
    __syncthreads();
#pragma unroll 1
    for (int base = G.g * kWave; base < k; base += kG * kWave) {
      const uint32_t i = static_cast<uint32_t>(base + G.lane);
      out.store_entry(i, area[i], area[ke + i]);
    }
  }
};

// One specified step of the capped search over the row (capped_step, with
// a row-wide count): false once the search has stopped. Every wave holds the
// same bracket, so all of them count (and reach the exchange) alike.
template <bool EPS0, int Q>
__device__ __forceinline__ bool row_capped_step(Group& G, const float (&v)[Q],
                                                CappedState& b, const SelectArgs& a) {
  if (!(b.steps < static_cast<uint32_t>(a.max_iter))) return false;
  if constexpr (!EPS0) {
    if (ballot(b.hi - b.lo > a.eps) == 0) return false;
  }
  const float mid = 0.5f * b.lo + 0.5f * b.hi;
  if ((ballot(b.lo < mid) & ballot(mid < b.hi)) == 0) return false;
  const int c = row_count(G, v, mid);
  ++b.steps;
  b.lo = c >= a.k ? mid : b.lo;
  b.hi = c <= a.k ? mid : b.hi;
  return true;
}

// The capped search (capped_row) on a row held by the group. The row's
// minimum, maximum and sum of squares are combined across the waves; the
// elements at or above the exact search's first threshold t0 are staged;
// when their count lands in the window every wave runs the specified steps
// on the row's candidate list (each midpoint at or above t0 gets the row's
// count, each below it takes the c > k branch as the row's count would),
// then the tie fill: over the candidates when lo >= t0 (wave 0 stores);
// else wave 0's split fill when its columns hold B's quota; else over the
// row, assembled in the candidate areas. When the first count misses the
// window the steps count over the whole row.
template <int Q, bool FULL, int QC, typename Out>
__device__ __forceinline__ void row_capped(Group& G, const float (&vin)[Q],
                                           const SelectArgs& a, int m_local, int col0,
                                           uint32_t* __restrict__ areas,
                                           const Out& out) {
  const int k = a.k;
  const int lane = G.lane;
  float v[Q];
  float s2 = 0.0f;  // tail positions were read as 0
#pragma unroll
  for (int s = 0; s < Q; ++s) {
    v[s] = vin[s];
    if constexpr (QC > 0) s2 = fmaf(vin[s], vin[s], s2);
  }
  mask_tail<Q, FULL>(m_local, lane, v);
  float mn = kInf, mx = -kInf;
#pragma unroll
  for (int s = 0; s < Q; ++s) {
    // Tail positions hold -inf (inputs are finite): out of the minimum.
    mn = fminf(mn, FULL || v[s] > -kInf ? v[s] : kInf);
    mx = fmaxf(mx, v[s]);
  }
  wave_reduce3<OpMin, OpMax, OpAdd>(mn, mx, s2);
  {
    uint32_t mns[kG], mxs[kG];
    G.exchange2(__float_as_uint(mn), __float_as_uint(mx), mns, mxs);
    mn = kInf;
    mx = -kInf;
#pragma unroll
    for (int i = 0; i < kG; ++i) {
      mn = fminf(mn, __uint_as_float(mns[i]));
      mx = fmaxf(mx, __uint_as_float(mxs[i]));
    }
  }
  const bool eps0 = a.eps == 0.0f;
  auto col = [lane, col0](int s) { return col0 + s * kWave + lane; };
  CappedState b{mn, mx, a.m, -1, 0u};
  if constexpr (QC > 0) {
    constexpr int kW = kWave * QC;
    s2 = row_sum_of_waves(G, s2);
    const float r = fminf(__builtin_amdgcn_sqrtf(s2), 1.0e35f);
    const float t0 = r * a.z_first;
    const int c0 = row_count_and_stage<Q, QC>(G, v, t0, col0, areas + G.g * 2 * sub_entries<QC>());
    if (c0 > k && c0 <= kW) {
      float cv[QC];
      int ci[QC];
      row_read_candidates<QC>(G, areas, c0, cv, ci);
      if (eps0) capped_run<true>(cv, b, a); else capped_run<false>(cv, b, a);
      auto cand_col = [&ci](int s) { return ci[s]; };
      if (ballot(b.lo >= t0) != 0) {
        // Every element >= lo is a candidate: wave 0 alone fills from them.
        if (G.g == 0) capped_emit<false>(cv, cand_col, b, k, out, out, lane);
        return;
      }
      // lo < t0: A = {x >= hi} lies among the candidates (hi is the row
      // maximum or a midpoint whose count was at most k, both >= t0). When
      // wave 0's columns hold B's quota (the first k - |A| elements of
      // {lo <= x < hi}), wave 0 alone emits: the split fill of capped_row
      // over its slots, then the rest of A from the candidates. Otherwise
      // the fill runs over the whole row. (Also testing whether [lo, t0)
      // is empty, so that B too is among the candidates, cost more than it
      // saved: 5-6% slower at k = 32 to 128 on rows with few distinct
      // values.)
      const int nA = count_ge(cv, b.hi);
      if (nA >= k) {
        if (G.g == 0) capped_emit<false>(cv, cand_col, b, k, out, out, lane);
        return;
      }
      uint32_t met_flag = 0;
      if (G.g == 0) {
        int nb = 0;
#pragma unroll
        for (int s = 0; s < Q; ++s)
          nb += popc(ballot(v[s] >= b.lo) & ~ballot(v[s] >= b.hi));
        met_flag = nb >= k - nA ? 1u : 0u;
      }
      uint32_t met[kG];
      G.exchange1(met_flag, met);
      if (met[0] != 0) {
        if (G.g == 0) emit_fill_split(v, cv, ci, lane, b.lo, b.hi, k, nA, out);
      } else {
        // Straight from each slot, every wave would store each 128-byte
        // output line in parts.
        const GroupStaged staged(areas, k, G.g, lane);
        row_emit_fill(G, v, col, b.lo, b.hi, k, staged);
        staged.flush(G, out, k);
      }
      return;
    }
  }
#pragma unroll 1
  while (eps0 ? row_capped_step<true>(G, v, b, a) : row_capped_step<false>(G, v, b, a)) {
  }
  if constexpr (QC > 0) {
    // The candidate areas hold k + 256 entries per array (64 QC >= 2k).
    const GroupStaged staged(areas, k, G.g, lane);
    row_emit_fill(G, v, col, b.lo, b.hi, k, staged);
    staged.flush(G, out, k);
  } else {
    row_emit_fill(G, v, col, b.lo, b.hi, k, out);
  }
}

// The kernel: block b takes rows b, b + gridDim.x, ... (a persistent grid);
// wave g of the block holds its quarter of each.
template <int Q, bool FULL, int QC, bool CAPPED, typename IdxT>
__global__ __launch_bounds__(kWave * kG) void rows_in_group(SelectArgs a) {
  constexpr int kE = sub_entries<QC>();
  __shared__ uint32_t areas[kG * 2 * kE];
  __shared__ uint32_t xch[4 * kG + 2 * kWave];
  // Wave 0's area to assemble output rows emitted from the candidates.
  __shared__ uint32_t ostage[2 * out_entries<QC>()];
  Group G;
  G.lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  G.g = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  G.xch = xch;
  G.parity = 0;
  const int col0 = G.g * kWave * Q;
  // This wave's part of the row length. Read back as a scalar: the code
  // generator otherwise keeps it per lane, where the per-slot tests of
  // mask_tail cannot take it.
  const int m_local = __builtin_amdgcn_readfirstlane(max(0, min(a.m - col0, kWave * Q)));
  const int lane = G.lane;
#pragma unroll 1
  for (int64_t r = blockIdx.x; r < a.n; r += gridDim.x) {
    // The lane index passes through an empty asm once per row, so that the
    // column of every slot is formed where it is used rather than kept in a
    // register of its own across the row loop (one register per slot).
    G.lane = lane;
    asm volatile("" : "+v"(G.lane));
    float v[Q];
    load_row<Q, FULL>(a.x + r * a.m + col0, m_local, G.lane, v);
    const OutRow<IdxT, Mode::kExact> out(a.out_val + r * a.k,
                                         static_cast<IdxT*>(a.out_idx) + r * a.k, a.k,
                                         nullptr, 0u, 0);
    if constexpr (CAPPED)
      row_capped<Q, FULL, QC>(G, v, a, m_local, col0, areas, out);
    else
      row_exact<Q, FULL, QC>(G, v, a, m_local, col0, areas, out, ostage);
    // The next row's candidates may be written while a slow wave still
    // reads this row's.
    __syncthreads();
  }
}

template <int Q, bool FULL, bool CAPPED, typename IdxT>
RowsKernel group_kernel_qc(int qc) {
  switch (qc) {
    case 1: return rows_in_group<Q, FULL, 1, CAPPED, IdxT>;
    case 2: return rows_in_group<Q, FULL, 2, CAPPED, IdxT>;
    case 4: return rows_in_group<Q, FULL, 4, CAPPED, IdxT>;
    case 8: return rows_in_group<Q, FULL, 8, CAPPED, IdxT>;
    default: return rows_in_group<Q, FULL, 0, CAPPED, IdxT>;
  }
}

}  // namespace group_detail

// The exact (or capped) kernel for rows of up to 4*64*Q columns held by a
// group of four waves, Q slots per lane per wave. full: the row length is
// exactly 4*64*Q.
template <int Q>
RowsKernel group_kernel(bool full, bool u8_index, int qc, bool capped) {
  using group_detail::group_kernel_qc;
  if (u8_index) return nullptr;
  if (capped)
    return full ? group_kernel_qc<Q, true, true, int32_t>(qc)
                : group_kernel_qc<Q, false, true, int32_t>(qc);
  return full ? group_kernel_qc<Q, true, false, int32_t>(qc)
              : group_kernel_qc<Q, false, false, int32_t>(qc);
}

}  // namespace rtopk
