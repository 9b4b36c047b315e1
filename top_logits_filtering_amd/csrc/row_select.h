// Threshold search for one row, written once against an abstract "source" of
// (raw value, original index) pairs. A source provides
//     template <class F> __device__ void for_each(F&& f) const;
// which calls f(raw, idx) for every element it holds, spread over the block's
// threads. Sources used: the row re-read from global memory, the row resident
// in registers, and a candidate list compacted into shared memory.
//
// The search follows the filter's steps (ApplyTopKTopPWithSorted guide, §2):
//   steps 1-3  -> k-th largest key by radix selection, counted with
//                 multiplicity, so every value equal to it survives;
//   steps 4-6  -> the top-p boundary, found by radix selection on probability
//                 mass: walking the stable order from the top, a position
//                 survives while the mass strictly above it is below
//                 (1 - t) * Z; inside the final run of equal values the higher
//                 original indices come first (stable ascending sort, §6.1),
//                 so the survivors of that run are its highest indices;
//   step 6 tail -> the top position (maximum value, highest index) always
//                 survives.
#pragma once

#include "device_common.h"

namespace tkp {

// k-th largest (1-based, with multiplicity) of keyfn(raw, idx) over the
// elements with pred(raw, idx), by 8-bit digits from the top. key_bits is a
// multiple of 8. Every thread of the block must call it.
template <class Src, class KeyFn, class Pred>
__device__ __forceinline__ uint32_t radix_select_desc(const Src& src, int key_bits, uint32_t k, KeyFn keyfn, Pred pred,
                                      RowSmem& sm) {
  uint32_t prefix = 0, pmask = 0;
  for (int shift = key_bits - 8; shift >= 0; shift -= 8) {
    clear_hists(sm, false);
    src.for_each([&](auto raw, int idx) {
      uint32_t key = keyfn(raw, idx);
      if ((key & pmask) == prefix && pred(raw, idx)) atomicAdd(&sm.hist[(key >> shift) & 255u], 1u);
    });
    __syncthreads();
    select_bin_count(sm, k);
    const uint32_t bin = static_cast<uint32_t>(sm.sel_bin);
    k -= sm.sel_above;
    prefix |= bin << shift;
    pmask |= 0xFFu << shift;
  }
  return prefix;
}

// Key of the maximum and the highest original index holding it.
template <class DT, class Src>
__device__ __forceinline__ void top_position(const Src& src, RowSmem& sm, uint32_t& K, uint32_t& I) {
  uint32_t kmax = 0;
  src.for_each([&](auto raw, int) {
    uint32_t key = DT::key(raw);
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

// Top-p boundary among the elements with key >= Kk (the top-k survivors).
// thr (1 <= thr <= Z) is the fixed-point threshold (1 - t) * Z, m the row
// maximum. Returns (Kp, Ip): survivors are key > Kp, or key == Kp with
// idx >= Ip.
// With with_index == false only Kp is computed (Ip = 0), which is enough when
// the result is used as a lower bound on the boundary key.
template <class DT, class Src>
__device__ __forceinline__ void topp_boundary(const Src& src, uint32_t Kk, float m, uint64_t thr, RowSmem& sm, uint32_t& Kp,
                              uint32_t& Ip, bool with_index = true) {
  uint32_t prefix = 0, pmask = 0;
  uint64_t acc = 0;  // mass strictly above the current prefix range
  for (int shift = DT::kKeyBits - 8; shift >= 0; shift -= 8) {
    clear_hists(sm, true);
    src.for_each([&](auto raw, int) {
      uint32_t key = DT::key(raw);
      if (key >= Kk && (key & pmask) == prefix) {
        uint32_t bin = (key >> shift) & 255u;
        atomicAdd(&sm.mhist[bin], mass_fx(DT::value(raw), m));
        atomicAdd(&sm.hist[bin], 1u);
      }
    });
    __syncthreads();
    select_bin_mass(sm, thr - acc);
    acc += sm.sel_above64;
    prefix |= static_cast<uint32_t>(sm.sel_bin) << shift;
    pmask |= 0xFFu << shift;
  }
  Kp = prefix;
  // Every element of the final run has the same value, hence the same mass.
  const uint32_t cnt = sm.sel_cnt;
  const uint64_t eg = sm.sel_mass / (cnt ? cnt : 1u);
  const uint64_t need = thr - acc;  // >= 1
  uint64_t ns64 = eg ? (need + eg - 1) / eg : cnt;
  uint32_t ns = ns64 >= cnt ? cnt : static_cast<uint32_t>(ns64);
  if (ns < 1) ns = 1;
  __syncthreads();  // everyone has read sel_* before it is reused
  if (ns >= cnt || !with_index) {
    Ip = 0;
  } else {
    const uint32_t kp = Kp;
    Ip = radix_select_desc(
        src, 24, ns, [](auto, int idx) { return static_cast<uint32_t>(idx); },
        [kp](auto raw, int) { return DT::key(raw) == kp; }, sm);
  }
}

// Full threshold pair (K, I) of a row, every statistic computed from `src`.
template <class DT, class Src>
__device__ __forceinline__ void solve_row(const Src& src, const RowParams& rp, RowSmem& sm, uint32_t& K, uint32_t& I) {
  K = 0;
  I = 0;
  if (!rp.k_on && rp.pmode == kPNone) return;
  uint32_t Kk = 0;
  if (rp.k_on) {
    Kk = radix_select_desc(
        src, DT::kKeyBits, rp.k, [](auto raw, int) { return DT::key(raw); }, [](auto, int) { return true; },
        sm);
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
  topp_boundary<DT>(src, Kk, m, thr, sm, K, I);
}

}  // namespace tkp
