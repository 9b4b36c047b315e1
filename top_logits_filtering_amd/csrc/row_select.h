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
// bin, and the range shrinks to that bin. A range under 1024 keys is settled
// in a single pass; a full 32-bit range takes four.
#pragma once

#include "device_common.h"

namespace tkp {

constexpr int kBinBits = 10;
constexpr int kBins = 1 << kBinBits;  // == kThreads: one bin per thread in the scans
static_assert(kBins == kThreads, "bin scans assume one bin per thread");

struct SelSmem {
  uint32_t cnt[kBins];
  uint64_t mass[kBins];
  uint32_t wtot32[kWaves];
  uint64_t wtot64[kWaves];
  int bin;
  uint32_t above;
  uint64_t above64;
  uint32_t bcnt;
  uint64_t bmass;
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
  __syncthreads();
  // totals of the waves before this one: lane i < w contributes wave i's total
  const uint32_t base = wave_sum_u32(l < w ? wtot[l] : 0u);
  return v + base;
}

__device__ __forceinline__ uint64_t block_incl_scan_u64(uint64_t v, uint64_t* wtot) {
  const int l = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
  v = wave_incl_scan_u64(v);
  if (l == kWave - 1) wtot[w] = v;
  __syncthreads();
  const uint64_t base = wave_sum_u64(l < w ? wtot[l] : 0ull);
  return v + base;
}

__device__ __forceinline__ void sel_clear(SelSmem& ss, bool with_mass) {
  ss.cnt[threadIdx.x] = 0;
  if (with_mass) ss.mass[threadIdx.x] = 0;
  __syncthreads();
}

// Walks the bins from the highest down (thread t owns bin kBins-1-t) and
// selects the first bin whose inclusive running count reaches target >= 1.
// If the target exceeds the total, bin 0 is selected. Result in ss.bin,
// ss.above (count strictly above), ss.bcnt; visible after the call.
__device__ __forceinline__ void sel_pick_count(SelSmem& ss, uint32_t target) {
  const int b = kBins - 1 - static_cast<int>(threadIdx.x);
  const uint32_t c = ss.cnt[b];
  const uint32_t incl = block_incl_scan_u32(c, ss.wtot32);
  const uint32_t excl = incl - c;
  if ((excl < target && target <= incl) || (b == 0 && target > incl)) {
    ss.bin = b;
    ss.above = excl;
    ss.bcnt = c;
  }
  __syncthreads();
}

// The same on the mass histogram: first bin whose running mass reaches
// target >= 1; also reports the bin's count and mass.
__device__ __forceinline__ void sel_pick_mass(SelSmem& ss, uint64_t target) {
  const int b = kBins - 1 - static_cast<int>(threadIdx.x);
  const uint64_t c = ss.mass[b];
  const uint64_t incl = block_incl_scan_u64(c, ss.wtot64);
  const uint64_t excl = incl - c;
  if ((excl < target && target <= incl) || (b == 0 && target > incl)) {
    ss.bin = b;
    ss.above64 = excl;
    ss.bmass = c;
    ss.bcnt = ss.cnt[b];
  }
  __syncthreads();
}

// k-th largest (1-based, with multiplicity) of keyfn(raw, idx) over the
// elements with pred(raw, idx), given that all of them lie in [lo, hi].
// Every thread of the block must call it.
template <class Src, class KeyFn, class Pred>
__device__ __forceinline__ uint32_t kth_largest_key(const Src& src, uint32_t k, uint32_t lo, uint32_t hi,
                                                    KeyFn keyfn, Pred pred, SelSmem& ss) {
  for (;;) {
    const uint32_t range = hi - lo;
    if (range == 0) return lo;
    const int shift = shift_for_range(range);
    sel_clear(ss, false);
    src.for_each([&](auto raw, int idx) {
      const uint32_t key = keyfn(raw, idx);
      if (key >= lo && key <= hi && pred(raw, idx)) atomicAdd(&ss.cnt[(key - lo) >> shift], 1u);
    });
    __syncthreads();
    sel_pick_count(ss, k);
    const uint32_t bin = static_cast<uint32_t>(ss.bin);
    k -= ss.above;
    const uint32_t nlo = lo + (bin << shift);
    const uint32_t span = (shift == 0) ? 0u : ((1u << shift) - 1u);
    hi = (hi - nlo > span) ? nlo + span : hi;
    lo = nlo;
    if (shift == 0) return lo;
  }
}

// Coarse lower bound for the k-th largest key: one histogram pass over
// [lo, hi]; gives the lower edge of the bin holding the k-th largest. Returns
// false when fewer than k elements lie in [lo, hi].
template <class Src, class KeyFn>
__device__ __forceinline__ bool kth_largest_bound(const Src& src, uint32_t k, uint32_t lo, uint32_t hi,
                                                  KeyFn keyfn, SelSmem& ss, uint32_t& bound) {
  const int shift = shift_for_range(hi - lo);
  sel_clear(ss, false);
  src.for_each([&](auto raw, int idx) {
    const uint32_t key = keyfn(raw, idx);
    if (key >= lo && key <= hi) atomicAdd(&ss.cnt[(key - lo) >> shift], 1u);
  });
  __syncthreads();
  sel_pick_count(ss, k);
  const bool ok = !(ss.bin == 0 && ss.above + ss.bcnt < k);
  bound = lo + (static_cast<uint32_t>(ss.bin) << shift);
  __syncthreads();
  return ok;
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
template <class DT, class Src>
__device__ __forceinline__ void topp_boundary(const Src& src, uint32_t lo, uint32_t hi, float m, uint64_t thr,
                                              int V, SelSmem& ss, uint32_t& Kp, uint32_t& Ip) {
  uint64_t acc = 0;  // mass strictly above the current range
  uint32_t cnt = 0;
  uint64_t bmass = 0;
  for (;;) {
    const int shift = shift_for_range(hi - lo);
    sel_clear(ss, true);
    src.for_each([&](auto raw, int) {
      const uint32_t key = DT::key(raw);
      if (key >= lo && key <= hi) {
        const uint32_t bin = (key - lo) >> shift;
        atomicAdd(&ss.mass[bin], mass_fx(DT::value(raw), m));
        atomicAdd(&ss.cnt[bin], 1u);
      }
    });
    __syncthreads();
    sel_pick_mass(ss, thr - acc);
    acc += ss.above64;
    cnt = ss.bcnt;
    bmass = ss.bmass;
    const uint32_t nlo = lo + (static_cast<uint32_t>(ss.bin) << shift);
    const uint32_t span = (shift == 0) ? 0u : ((1u << shift) - 1u);
    hi = (hi - nlo > span) ? nlo + span : hi;
    lo = nlo;
    __syncthreads();
    if (shift == 0) break;
  }
  Kp = lo;
  // Every element of the final run has the same value, hence the same mass.
  const uint64_t eg = bmass / (cnt ? cnt : 1u);
  const uint64_t need = thr - acc;  // >= 1
  const uint64_t ns64 = eg ? (need + eg - 1) / eg : cnt;
  uint32_t ns = ns64 >= cnt ? cnt : static_cast<uint32_t>(ns64);
  if (ns < 1) ns = 1;
  if (ns >= cnt) {
    Ip = 0;
  } else {
    const uint32_t kp = Kp;
    Ip = kth_largest_key(
        src, ns, 0u, static_cast<uint32_t>(V - 1), [](auto, int idx) { return static_cast<uint32_t>(idx); },
        [kp](auto raw, int) { return DT::key(raw) == kp; }, ss);
  }
}

// Coarse lower bound for the top-p boundary: one mass histogram over
// [lo, hi]; gives the lower edge of the bin where the running mass from the
// top reaches thr. Returns false when the whole range carries less than thr.
template <class DT, class Src>
__device__ __forceinline__ bool topp_bound(const Src& src, uint32_t lo, uint32_t hi, float m, uint64_t thr,
                                           SelSmem& ss, uint32_t& bound) {
  const int shift = shift_for_range(hi - lo);
  sel_clear(ss, true);
  src.for_each([&](auto raw, int) {
    const uint32_t key = DT::key(raw);
    if (key >= lo && key <= hi) {
      const uint32_t bin = (key - lo) >> shift;
      atomicAdd(&ss.mass[bin], mass_fx(DT::value(raw), m));
      atomicAdd(&ss.cnt[bin], 1u);
    }
  });
  __syncthreads();
  sel_pick_mass(ss, thr);
  const bool ok = !(ss.bin == 0 && ss.above64 + ss.bmass < thr);
  bound = lo + (static_cast<uint32_t>(ss.bin) << shift);
  __syncthreads();
  return ok;
}

// Full threshold pair (K, I) of a row, every statistic computed from `src`,
// which holds all V elements of the row.
template <class DT, class Src>
__device__ __forceinline__ void solve_row(const Src& src, const RowParams& rp, int V, RowSmem& sm, SelSmem& ss,
                                          uint32_t& K, uint32_t& I) {
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
  float mloc = -INFINITY;
  src.for_each([&](auto raw, int) { mloc = fmaxf(mloc, DT::value(raw)); });
  const float m = block_max_f32(mloc, sm);
  uint64_t zloc = 0;
  src.for_each([&](auto raw, int) {
    if (DT::key(raw) >= Kk) zloc += mass_fx(DT::value(raw), m);
  });
  const uint64_t Z = block_sum_u64(zloc, sm);
  const uint64_t thr = topp_threshold(rp.t, Z);
  if (thr == 0) {
    top_position<DT>(src, sm, K, I);
    return;
  }
  topp_boundary<DT>(src, Kk, kKeyMax, m, thr, V, ss, K, I);
}

}  // namespace tkp
