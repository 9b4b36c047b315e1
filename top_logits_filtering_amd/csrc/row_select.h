// Threshold search for one row, written once against an abstract "source" of
// (raw value, original index) pairs. A source provides
//     template <class F> __device__ void for_each(F&& f) const;
// which calls f(raw, idx) for every element it holds, spread over the block's
// threads. Sources used: the row re-read from global memory, and the
// candidate vectors gathered into shared memory.
//
// The search follows the filter's steps (ApplyTopKTopPWithSorted guide, §2):
//   steps 1-3  -> the k-th largest key, counted with multiplicity, so every
//                 value equal to it survives;
//   steps 4-6  -> the top-p boundary: walking the stable order from the top, a
//                 position survives while the probability mass strictly above
//                 it is below (1 - t) * Z; inside the final run of equal values
//                 the higher original indices come first (stable ascending
//                 sort, §6.1), so the survivors of that run are its highest
//                 indices;
//   step 6 tail -> the top position (maximum value, highest index) always
//                 survives.
//
// Selection is a range-adaptive radix search: with every candidate key known
// to lie in [lo, hi], one pass histograms (key - lo) >> shift into at most
// 1024 bins (shift chosen so the range fits), one block-wide scan picks the
// bin, and the range shrinks to the smallest and largest key actually present
// in that bin (each pass also records them per bin). A range under 1024 keys
// is settled in a single pass, and so is any range whose picked bin holds a
// single distinct key (equal values, or few elements spread over a wide
// range); a full 32-bit range takes at most four.
#pragma once

#include "device_common.h"

namespace tkp {

constexpr int kBinBits = 10;
constexpr int kBins = 1 << kBinBits;  // == kThreads: one bin per thread in the scans
static_assert(kBins == kThreads, "bin scans assume one bin per thread");

struct alignas(16) SelSmem {
  alignas(16) uint32_t cnt[kBins];
  alignas(16) uint64_t mass[kBins];
  // per bin, the largest key and the largest complemented key (so the
  // smallest key is ~knmn): both start at zero like the counts
  alignas(16) uint32_t kmx[kBins];
  alignas(16) uint32_t knmn[kBins];
  uint32_t wtot32[kWaves];
  uint64_t wtot64[kWaves];
  int bin;
  uint32_t above;
  uint64_t above64;
  uint32_t bcnt;
  uint64_t bmass;
  uint32_t bkmin, bkmax;  // smallest and largest key in the picked bin (passes that record them)
  int kbin;      // joint pick: bin of the k-th largest
  uint64_t thr;  // joint pick: fixed-point top-p threshold over the top-k survivors
  uint32_t run_n;              // boundary run gathered for one-wave ranking (zero between uses)
  uint32_t run_idx[kWave];     // its indices
  uint32_t run_res;
};

__device__ __forceinline__ int shift_for_range(uint32_t range) {
  const int bits = range == 0 ? 0 : 32 - __clz(range);
  return bits > kBinBits ? bits - kBinBits : 0;
}

// Inclusive prefix sum over threadIdx.x (u32 / u64).
__device__ __forceinline__ uint32_t block_incl_scan_u32(uint32_t v, uint32_t* wtot) {
  const int l = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  v = wave_incl_scan_u32(v);
  if (l == kWave - 1) wtot[w] = v;
  lds_barrier();
  // totals of the waves before this one: lane i < w contributes wave i's total
  const uint32_t base = wave_sum_u32(l < w ? wtot[l] : 0u);
  return v + base;
}

__device__ __forceinline__ uint64_t block_incl_scan_u64(uint64_t v, uint64_t* wtot) {
  const int l = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  v = wave_incl_scan_u64(v);
  if (l == kWave - 1) wtot[w] = v;
  lds_barrier();
  const uint64_t base = wave_sum_u64(l < w ? wtot[l] : 0ull);
  return v + base;
}

// The histograms are kept all-zero between passes: they are cleared once
// (sel_reset, before a barrier) and every pick clears what it read, so a pass
// costs one barrier after its histogram and one after its pick.
__device__ __forceinline__ void sel_reset(SelSmem& ss) {
  ss.cnt[threadIdx.x] = 0;
  ss.mass[threadIdx.x] = 0;
  ss.kmx[threadIdx.x] = 0;
  ss.knmn[threadIdx.x] = 0;
  if (threadIdx.x == 0) ss.run_n = 0;
}

// A histogram pass that records key ranges calls this for each element.
__device__ __forceinline__ void sel_note_key(SelSmem& ss, uint32_t bin, uint32_t key) {
  atomicMax(&ss.kmx[bin], key);
  atomicMax(&ss.knmn[bin], ~key);
}

// Bins per lane when one wave scans the whole histogram: lane l owns the 16
// consecutive bins [kBins - 16 (l + 1), kBins - 16 l), so lanes run from the
// highest bins down. The pick takes two levels: a wave scan of the lanes'
// sums finds the lane L holding the target, then the 16 lanes of a DPP row
// each take one of L's bins (from its top) and a row scan finds the bin.
constexpr int kPickSpan = kBins / kWave;
static_assert(kPickSpan == 16, "pick layout assumes 16 bins per lane");

// Inclusive prefix sums over the 16 lanes of each DPP row.
__device__ __forceinline__ uint32_t row_incl_scan_u32(uint32_t v) {
  v += dpp_u32<dpp::kRowShr1>(v, 0u);
  v += dpp_u32<dpp::kRowShr2>(v, 0u);
  v += dpp_u32<dpp::kRowShr4>(v, 0u);
  v += dpp_u32<dpp::kRowShr8>(v, 0u);
  return v;
}
__device__ __forceinline__ uint64_t row_incl_scan_u64(uint64_t v) {
  v += dpp_u64<dpp::kRowShr1>(v, 0ull);
  v += dpp_u64<dpp::kRowShr2>(v, 0ull);
  v += dpp_u64<dpp::kRowShr4>(v, 0ull);
  v += dpp_u64<dpp::kRowShr8>(v, 0ull);
  return v;
}

// Zeroes the range arrays over one pick lane's bins [base, base + 16).
__device__ __forceinline__ void sel_clear_ranges(SelSmem& ss, int base) {
  const vec_t z = {0u, 0u, 0u, 0u};
  vec_t* xw = reinterpret_cast<vec_t*>(&ss.kmx[base]);
  vec_t* nw = reinterpret_cast<vec_t*>(&ss.knmn[base]);
#pragma unroll
  for (int q = 0; q < kPickSpan / 4; ++q) {
    xw[q] = z;
    nw[q] = z;
  }
}

// Walks the bins from the highest down and selects the first bin whose
// inclusive running count reaches target >= 1; if the target exceeds the
// total, bin 0 is selected. Result in ss.bin, ss.above (count strictly
// above) and ss.bcnt, visible after the call. Wave 0 scans (the histogram
// must be complete: callers place a barrier before) and clears the bins.
// LEAN keeps the histogram reads two at a time (for steps where the row tile
// still occupies most registers); otherwise all of a lane's bins are read at
// once, so the scan waits for one shared-memory round trip instead of several.
// RANGES: the pass recorded key ranges (sel_note_key); the picked bin's range
// goes to ss.bkmin / ss.bkmax and the range arrays are cleared too.
template <bool LEAN = false, bool RANGES = false>
__device__ __forceinline__ void sel_pick_count(SelSmem& ss, uint32_t target) {
  if (threadIdx.x < kWave) {
    const int l = static_cast<int>(threadIdx.x);
    const int base = kBins - kPickSpan * (l + 1);
    const vec_t* cv = reinterpret_cast<const vec_t*>(&ss.cnt[base]);
    uint32_t sum = 0;
    if constexpr (LEAN) {
#pragma unroll 2
      for (int q = 0; q < kPickSpan / 4; ++q) {
        const vec_t c4 = cv[q];
        sum += c4.x + c4.y + c4.z + c4.w;
      }
    } else {
      vec_t c4[kPickSpan / 4];
#pragma unroll
      for (int q = 0; q < kPickSpan / 4; ++q) c4[q] = cv[q];
#pragma unroll
      for (int q = 0; q < kPickSpan / 4; ++q) sum += c4[q].x + c4[q].y + c4[q].z + c4[q].w;
    }
    const uint32_t incl = wave_incl_scan_u32(sum);
    const uint32_t total = lane63_u32(incl);
    const bool short_total = target > total;  // then bin 0, the lowest bin of lane 63
    const uint64_t hitm = __ballot(incl - sum < target && target <= incl);
    const int L = short_total ? kWave - 1 : __ffsll(static_cast<unsigned long long>(hitm)) - 1;
    const uint32_t exclL = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl - sum), L));
    // second level: lane r of each row takes bin (top of L's range) - r
    const int r = l & 15;
    const int binr = kBins - kPickSpan * L - 1 - r;
    const uint32_t c = ss.cnt[binr];
    const uint32_t rin = row_incl_scan_u32(c);
    const uint32_t t2 = target - exclL;
    const uint64_t hit2 = __ballot(l < 16 && rin - c < t2 && t2 <= rin);
    const int R = short_total ? 15 : __ffsll(static_cast<unsigned long long>(hit2)) - 1;
    if (l == R) {
      ss.bin = binr;
      ss.above = exclL + rin - c;
      ss.bcnt = c;
      if constexpr (RANGES) {
        ss.bkmax = ss.kmx[binr];
        ss.bkmin = ~ss.knmn[binr];
      }
    }
    const vec_t z = {0u, 0u, 0u, 0u};
    vec_t* cw = reinterpret_cast<vec_t*>(&ss.cnt[base]);
#pragma unroll
    for (int q = 0; q < kPickSpan / 4; ++q) cw[q] = z;
    if constexpr (RANGES) sel_clear_ranges(ss, base);
  }
  lds_barrier();
}

// The same on the mass histogram: first bin whose running mass reaches
// target >= 1; also reports the bin's count and mass. Clears both histograms.
template <bool LEAN = false, bool RANGES = false>
__device__ __forceinline__ void sel_pick_mass(SelSmem& ss, uint64_t target) {
  if (threadIdx.x < kWave) {
    const int l = static_cast<int>(threadIdx.x);
    const int base = kBins - kPickSpan * (l + 1);
    const vec_t* mv = reinterpret_cast<const vec_t*>(&ss.mass[base]);  // two u64 per vector
    uint64_t sum = 0;
    if constexpr (LEAN) {
#pragma unroll 2
      for (int q = 0; q < kPickSpan / 2; ++q) {
        const vec_t m2 = mv[q];
        sum += (static_cast<uint64_t>(m2.y) << 32 | m2.x) + (static_cast<uint64_t>(m2.w) << 32 | m2.z);
      }
    } else {
      vec_t m2[kPickSpan / 2];
#pragma unroll
      for (int q = 0; q < kPickSpan / 2; ++q) m2[q] = mv[q];
#pragma unroll
      for (int q = 0; q < kPickSpan / 2; ++q)
        sum += (static_cast<uint64_t>(m2[q].y) << 32 | m2[q].x) + (static_cast<uint64_t>(m2[q].w) << 32 | m2[q].z);
    }
    const uint64_t incl = wave_incl_scan_u64(sum);
    const uint64_t total = lane63_u64(incl);
    const bool short_total = target > total;
    const uint64_t hitm = __ballot(incl - sum < target && target <= incl);
    const int L = short_total ? kWave - 1 : __ffsll(static_cast<unsigned long long>(hitm)) - 1;
    const uint64_t ex = incl - sum;
    const uint64_t exclL = static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(ex >> 32), L))) << 32 |
                           static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(ex), L));
    const int r = l & 15;
    const int binr = kBins - kPickSpan * L - 1 - r;
    const uint64_t c = ss.mass[binr];
    const uint64_t rin = row_incl_scan_u64(c);
    const uint64_t t2 = target - exclL;
    const uint64_t hit2 = __ballot(l < 16 && rin - c < t2 && t2 <= rin);
    const int R = short_total ? 15 : __ffsll(static_cast<unsigned long long>(hit2)) - 1;
    if (l == R) {
      ss.bin = binr;
      ss.above64 = exclL + rin - c;
      ss.bmass = c;
      ss.bcnt = ss.cnt[binr];
      if constexpr (RANGES) {
        ss.bkmax = ss.kmx[binr];
        ss.bkmin = ~ss.knmn[binr];
      }
    }
    const vec_t z = {0u, 0u, 0u, 0u};
    vec_t* mw = reinterpret_cast<vec_t*>(&ss.mass[base]);
#pragma unroll
    for (int q = 0; q < kPickSpan / 2; ++q) mw[q] = z;
    vec_t* cw = reinterpret_cast<vec_t*>(&ss.cnt[base]);
#pragma unroll
    for (int q = 0; q < kPickSpan / 4; ++q) cw[q] = z;
    if constexpr (RANGES) sel_clear_ranges(ss, base);
  }
  lds_barrier();
}

// Top-k and top-p together from one pass of both histograms over a range
// where each bin holds a single key: the bin of the k-th largest (count from
// the top reaches k; the histogram must hold at least k elements), Z = the
// mass of that bin and every bin above it, thr = ceil((1 - t) Z), and, when
// thr > 0, the first bin from the top whose running mass reaches thr, with the
// mass strictly above it, its mass and its count (ss.bin, ss.above64,
// ss.bmass, ss.bcnt). ss.kbin and ss.thr hold the others. Wave 0 works and
// clears both histograms.
__device__ __forceinline__ void sel_pick_joint(SelSmem& ss, uint32_t k, float t) {
  if (threadIdx.x < kWave) {
    const int l = static_cast<int>(threadIdx.x);
    const int base = kBins - kPickSpan * (l + 1);
    const vec_t* cv = reinterpret_cast<const vec_t*>(&ss.cnt[base]);
    const vec_t* mv = reinterpret_cast<const vec_t*>(&ss.mass[base]);
    vec_t c4[kPickSpan / 4], m2[kPickSpan / 2];
#pragma unroll
    for (int q = 0; q < kPickSpan / 4; ++q) c4[q] = cv[q];
#pragma unroll
    for (int q = 0; q < kPickSpan / 2; ++q) m2[q] = mv[q];
    uint32_t csum = 0;
#pragma unroll
    for (int q = 0; q < kPickSpan / 4; ++q) csum += c4[q].x + c4[q].y + c4[q].z + c4[q].w;
    uint64_t msum = 0;
#pragma unroll
    for (int q = 0; q < kPickSpan / 2; ++q)
      msum += (static_cast<uint64_t>(m2[q].y) << 32 | m2[q].x) + (static_cast<uint64_t>(m2[q].w) << 32 | m2[q].z);
    const uint32_t cin = wave_incl_scan_u32(csum);
    const uint64_t min = wave_incl_scan_u64(msum);
    const uint32_t cex = cin - csum;
    const uint64_t mex = min - msum;
    const int r = l & 15;
    // the k-th largest
    const uint64_t hk = __ballot(cex < k && k <= cin);
    const int Lk = hk ? __ffsll(static_cast<unsigned long long>(hk)) - 1 : kWave - 1;
    const int binrk = kBins - kPickSpan * Lk - 1 - r;
    const uint32_t ck = ss.cnt[binrk];
    const uint64_t mk = ss.mass[binrk];
    const uint32_t ckin = row_incl_scan_u32(ck);
    const uint64_t mkin = row_incl_scan_u64(mk);
    const uint32_t tk = k - readlane_u32(cex, Lk);
    const uint64_t hk2 = __ballot(l < 16 && ckin - ck < tk && tk <= ckin);
    const int Rk = hk2 ? __ffsll(static_cast<unsigned long long>(hk2)) - 1 : 15;
    const uint64_t Z = readlane_u64(mex, Lk) + readlane_u64(mkin, Rk);
    const uint64_t thr = topp_threshold(t, Z);
    if (l == 0) {
      ss.kbin = kBins - kPickSpan * Lk - 1 - Rk;
      ss.thr = thr;
    }
    // the top-p boundary: thr <= Z, so at or above the k-th largest's bin
    if (thr > 0) {
      const uint64_t hp = __ballot(mex < thr && thr <= min);
      const int Lp = __ffsll(static_cast<unsigned long long>(hp)) - 1;
      const uint64_t mexL = readlane_u64(mex, Lp);
      const int binrp = kBins - kPickSpan * Lp - 1 - r;
      const uint64_t mp = ss.mass[binrp];
      const uint64_t mpin = row_incl_scan_u64(mp);
      const uint64_t tp = thr - mexL;
      const uint64_t hp2 = __ballot(l < 16 && mpin - mp < tp && tp <= mpin);
      const int Rp = __ffsll(static_cast<unsigned long long>(hp2)) - 1;
      if (l == Rp) {
        ss.bin = binrp;
        ss.above64 = mexL + mpin - mp;
        ss.bmass = mp;
        ss.bcnt = ss.cnt[binrp];
      }
    }
    const vec_t z = {0u, 0u, 0u, 0u};
    vec_t* mw = reinterpret_cast<vec_t*>(&ss.mass[base]);
#pragma unroll
    for (int q = 0; q < kPickSpan / 2; ++q) mw[q] = z;
    vec_t* cw = reinterpret_cast<vec_t*>(&ss.cnt[base]);
#pragma unroll
    for (int q = 0; q < kPickSpan / 4; ++q) cw[q] = z;
  }
  lds_barrier();
}

// k-th largest (1-based, with multiplicity) of keyfn(raw, idx) over the
// elements with pred(raw, idx), given that all of them lie in [lo, hi].
// Every thread of the block must call it. With rem, *rem receives the rank
// of the k-th largest among the elements equal to it (k minus the count of
// larger ones), the same in every thread.
template <class Src, class KeyFn, class Pred>
__device__ __forceinline__ uint32_t kth_largest_key(const Src& src, uint32_t k, uint32_t lo, uint32_t hi,
                                                    KeyFn keyfn, Pred pred, SelSmem& ss,
                                                    uint32_t* rem = nullptr) {
  for (;;) {
    const uint32_t range = hi - lo;
    if (range == 0) {
      if (rem != nullptr) *rem = k;
      return lo;
    }
    const int shift = shift_for_range(range);
    if (shift == 0) {  // one key per bin: this pass settles it
      src.for_each([&](auto raw, int idx) {
        const uint32_t key = keyfn(raw, idx);
        if (key >= lo && key <= hi && pred(raw, idx)) atomicAdd(&ss.cnt[key - lo], 1u);
      });
      lds_barrier();
      sel_pick_count(ss, k);
      if (rem != nullptr) *rem = k - ss.above;
      return lo + static_cast<uint32_t>(ss.bin);
    }
    src.for_each([&](auto raw, int idx) {
      const uint32_t key = keyfn(raw, idx);
      if (key >= lo && key <= hi && pred(raw, idx)) {
        const uint32_t bin = (key - lo) >> shift;
        atomicAdd(&ss.cnt[bin], 1u);
        sel_note_key(ss, bin, key);
      }
    });
    lds_barrier();
    sel_pick_count<false, true>(ss, k);
    k -= ss.above;
    if (ss.bcnt != 0) {  // the keys present in the bin (it holds the k-th largest)
      lo = ss.bkmin;
      hi = ss.bkmax;
    } else {  // not reached when k is within the count: the bin's whole span
      lo += static_cast<uint32_t>(ss.bin) << shift;
      hi = (hi - lo > (1u << shift) - 1u) ? lo + ((1u << shift) - 1u) : hi;
    }
  }
}

// Coarse lower bound for the k-th largest key: one histogram pass over
// [lo, hi]; gives the lower edge of the bin holding the k-th largest. Returns
// false when fewer than k elements lie in [lo, hi].
template <class Src, class KeyFn>
__device__ __forceinline__ bool kth_largest_bound(const Src& src, uint32_t k, uint32_t lo, uint32_t hi,
                                                  KeyFn keyfn, SelSmem& ss, uint32_t& bound) {
  const int shift = shift_for_range(hi - lo);
  src.for_each([&](auto raw, int idx) {
    const uint32_t key = keyfn(raw, idx);
    if (key >= lo && key <= hi) atomicAdd(&ss.cnt[(key - lo) >> shift], 1u);
  });
  lds_barrier();
  sel_pick_count<true>(ss, k);
  const bool ok = !(ss.bin == 0 && ss.above + ss.bcnt < k);
  bound = lo + (static_cast<uint32_t>(ss.bin) << shift);
  return ok;
}

// Index threshold inside the final run of equal values at a top-p boundary:
// the run (key Kp, cnt elements of equal mass, bmass in total) is entered
// with `need` (>= 1) of the threshold still to reach; its members are taken
// from the highest index down until the mass strictly above the next one
// reaches the threshold. Returns Ip (survivors of the run: index >= Ip).
template <class DT, class Src>
__device__ __forceinline__ uint32_t boundary_index(const Src& src, uint32_t Kp, uint64_t need, uint32_t cnt,
                                                   uint64_t bmass, int V, SelSmem& ss) {
  if (cnt <= 1) return 0;  // a single element: it is the last survivor
  const uint64_t eg = bmass / cnt;
  const uint64_t ns64 = eg ? (need + eg - 1) / eg : cnt;
  uint32_t ns = ns64 >= cnt ? cnt : static_cast<uint32_t>(ns64);
  if (ns < 1) ns = 1;
  if (ns >= cnt) return 0;
  if (cnt <= static_cast<uint32_t>(kWave)) {
    // a short run: gather its indices and let wave 0 take the ns-th largest
    src.for_each([&](auto raw, int idx) {
      if (DT::key(raw) == Kp) ss.run_idx[atomicAdd(&ss.run_n, 1u)] = static_cast<uint32_t>(idx);
    });
    lds_barrier();
    if (threadIdx.x < kWave) {
      const int l = static_cast<int>(threadIdx.x);
      const int n = static_cast<int>(cnt);
      const uint32_t mine = l < n ? ss.run_idx[l] : 0u;
      uint32_t rank = 0;  // indices are distinct: larger ones come first
      for (int i = 0; i < n; ++i) rank += readlane_u32(mine, i) > mine ? 1u : 0u;
      if (l < n && rank == ns - 1) ss.run_res = mine;
      if (l == 0) ss.run_n = 0;
    }
    lds_barrier();
    return ss.run_res;
  }
  return kth_largest_key(
      src, ns, 0u, static_cast<uint32_t>(V - 1), [](auto, int idx) { return static_cast<uint32_t>(idx); },
      [Kp](auto raw, int) { return DT::key(raw) == Kp; }, ss);
}

// Key of the maximum and the highest original index holding it.
template <class DT, class Src>
__device__ __forceinline__ void top_position(const Src& src, RowSmem& sm, uint32_t& K, uint32_t& I) {
  uint32_t kmax = 0;
  src.for_each([&](auto raw, int) {
    const uint32_t key = DT::key(raw);
    kmax = key > kmax ? key : kmax;
  });
  kmax = block_max_u32(kmax, sm);
  uint32_t imax = 0;
  src.for_each([&](auto raw, int idx) {
    if (DT::key(raw) == kmax) imax = static_cast<uint32_t>(idx) > imax ? static_cast<uint32_t>(idx) : imax;
  });
  K = kmax;
  I = block_max_u32(imax, sm);
}

// Top-p boundary among the elements with key in [lo, hi], lo being the
// top-k threshold (or the smallest key when top-k is off). thr (1 <= thr <=
// the mass of those elements) is the fixed-point threshold (1 - t) * Z and m
// the row maximum. Gives (Kp, Ip): survivors are key > Kp, or key == Kp with
// idx >= Ip.
template <class DT, bool kWholeRow = false, class Src>
__device__ __forceinline__ void topp_boundary(const Src& src, uint32_t lo, uint32_t hi, float m, uint64_t thr,
                                              int V, SelSmem& ss, uint32_t& Kp, uint32_t& Ip) {
  uint64_t acc = 0;  // mass strictly above the current range
  uint32_t cnt = 0;
  uint64_t bmass = 0;
  for (;;) {
    const int shift = shift_for_range(hi - lo);
    // The keys present in each bin narrow the next pass, and end the search
    // when the picked bin holds one key. Passes over a whole row of 16-bit
    // keys skip that: a bin then spans at most 64 keys, which the next pass
    // resolves exactly either way, and two atomics per element are saved
    // (candidate lists hold a few elements per thread, where the pass that
    // a one-key bin saves is worth more).
    const bool ranges = shift != 0 && (DT::kKeyBits == 32 || !kWholeRow);
    src.for_each([&](auto raw, int) {
      const uint32_t key = DT::key(raw);
      if (key >= lo && key <= hi) {
        const uint32_t bin = (key - lo) >> shift;
        atomicAdd(&ss.mass[bin], mass_fx(DT::value(raw), m));
        atomicAdd(&ss.cnt[bin], 1u);
        if (ranges) sel_note_key(ss, bin, key);
      }
    });
    lds_barrier();
    if (!ranges)
      sel_pick_mass(ss, thr - acc);
    else
      sel_pick_mass<false, true>(ss, thr - acc);
    acc += ss.above64;
    cnt = ss.bcnt;
    bmass = ss.bmass;
    if (shift == 0) {
      lo += static_cast<uint32_t>(ss.bin);
      break;
    }
    if (ranges && cnt != 0) {  // the keys present in the bin (it holds the boundary)
      lo = ss.bkmin;
      hi = ss.bkmax;
    } else {  // the bin's whole span
      lo += static_cast<uint32_t>(ss.bin) << shift;
      hi = (hi - lo > (1u << shift) - 1u) ? lo + ((1u << shift) - 1u) : hi;
    }
    if (lo == hi) break;  // one key left: the bin's count and mass are its run
  }
  Kp = lo;
  // Every element of the final run has the same value, hence the same mass.
  Ip = boundary_index<DT>(src, Kp, thr - acc, cnt, bmass, V, ss);
}

// Coarse lower bound for the top-p boundary: one mass histogram over
// [lo, hi]; gives the lower edge of the bin where the running mass from the
// top reaches thr. Returns false when the whole range carries less than thr.
template <class DT, class Src>
__device__ __forceinline__ bool topp_bound(const Src& src, uint32_t lo, uint32_t hi, float m, uint64_t thr,
                                           SelSmem& ss, uint32_t& bound) {
  const int shift = shift_for_range(hi - lo);
  src.for_each([&](auto raw, int) {
    const uint32_t key = DT::key(raw);
    if (key >= lo && key <= hi) {
      const uint32_t bin = (key - lo) >> shift;
      atomicAdd(&ss.mass[bin], mass_fx(DT::value(raw), m));
      atomicAdd(&ss.cnt[bin], 1u);
    }
  });
  lds_barrier();
  sel_pick_mass<true>(ss, thr);
  const bool ok = !(ss.bin == 0 && ss.above64 + ss.bmass < thr);
  bound = lo + (static_cast<uint32_t>(ss.bin) << shift);
  return ok;
}

// Smallest key among the elements of `src` that survive min-p (m the row
// maximum). Every thread of the block must call it.
template <class DT, class Src>
__device__ __forceinline__ uint32_t min_p_key(const Src& src, float m, float minp, RowSmem& sm) {
  uint32_t nk = 0;  // largest complemented key, so the smallest key is ~nk
  src.for_each([&](auto raw, int) {
    if (min_p_keeps(DT::value(raw), m, minp)) {
      const uint32_t c = ~DT::key(raw);
      nk = c > nk ? c : nk;
    }
  });
  return ~block_max_u32(nk, sm);
}

// The min-p stage on top of a top-k / top-p pair: every stage keeps a suffix
// of the stable order, so the result is the larger pair in (key, index) order.
__device__ __forceinline__ void combine_min_p(uint32_t Kmp, uint32_t& K, uint32_t& I) {
  if (Kmp > K) {
    K = Kmp;
    I = 0;
  }
}

// Full threshold pair (K, I) of a row, every statistic computed from `src`,
// which holds all V elements of the row.
// What a caller already knows of a row: its maximum (m_ok), and for rows with
// top-p but no top-k the top-p threshold in 2^-43 units (thr != 0).
struct RowKnown {
  bool m_ok = false;
  float m = 0.0f;
  uint64_t thr = 0;
};

template <class DT, class Src>
__device__ __forceinline__ void solve_row_kp(const Src& src, const RowParams& rp, int V, RowSmem& sm, SelSmem& ss,
                                             uint32_t& K, uint32_t& I, const RowKnown& known) {
  K = 0;
  I = 0;
  if (!rp.k_on && rp.pmode == kPNone) return;
  constexpr uint32_t kKeyMax = DT::kKeyBits == 32 ? 0xFFFFFFFFu : ((1u << DT::kKeyBits) - 1u);
  uint32_t Kk = 0;
  if (rp.k_on) {
    Kk = kth_largest_key(
        src, rp.k, 0u, kKeyMax, [](auto raw, int) { return DT::key(raw); }, [](auto, int) { return true; }, ss);
  }
  if (rp.pmode == kPNone) {
    K = Kk;
    return;
  }
  if (rp.pmode == kPTopOnly) {
    top_position<DT>(src, sm, K, I);
    return;
  }
  float m;
  uint64_t thr;
  if (known.thr != 0 && !rp.k_on) {  // the row maximum and threshold were formed already
    m = known.m;
    thr = known.thr;
  } else {
    float mloc = -INFINITY;
    src.for_each([&](auto raw, int) { mloc = fmaxf(mloc, DT::value(raw)); });
    m = block_max_f32(mloc, sm);
    uint64_t zloc = 0;
    src.for_each([&](auto raw, int) {
      if (DT::key(raw) >= Kk) zloc += mass_fx(DT::value(raw), m);
    });
    const uint64_t Z = block_sum_u64(zloc, sm);
    thr = topp_threshold(rp.t, Z);
  }
  if (thr == 0) {
    top_position<DT>(src, sm, K, I);
    return;
  }
  topp_boundary<DT, true>(src, Kk, kKeyMax, m, thr, V, ss, K, I);
}

template <class DT, class Src>
__device__ __forceinline__ void solve_row(const Src& src, const RowParams& rp, int V, RowSmem& sm, SelSmem& ss,
                                          uint32_t& K, uint32_t& I, const RowKnown& known = RowKnown{}) {
  solve_row_kp<DT>(src, rp, V, sm, ss, K, I, known);
  if (rp.mp_on) {
    float m = known.m;
    if (!known.m_ok) {
      float mloc = -INFINITY;
      src.for_each([&](auto raw, int) { mloc = fmaxf(mloc, DT::value(raw)); });
      m = block_max_f32(mloc, sm);
    }
    combine_min_p(min_p_key<DT>(src, m, rp.minp, sm), K, I);
  }
}

}  // namespace tkp
