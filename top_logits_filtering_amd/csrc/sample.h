// Sampling after the filter: the "Subsequent processing" stage of Ascend's
// aclnnTopKTopPSampleV2 page. probs are the filtered probabilities in
// descending order (the reverse of the stable ascending order, so equal
// values take the higher original index first).
//   * None mode (no q): the index of the first maximum of probs, i.e. the
//     maximum value with the highest index.
//   * QSample: the index of the first maximum of probs / (q[r] + eps), q's
//     entry r pairing with descending rank r. Only survivors can win (masked
//     positions have zero probability), so each survivor's rank among the
//     survivors is all that is needed; the softmax normalisation is common to
//     every survivor and cancels, leaving exp(x - m) / (q[r] + eps).
// Ranks come from a counting sort over the survivors' keys: a histogram over
// [K, kmax] (range-adaptive 1024 bins), bin bases counted from the top, the
// survivors placed by bin into a shared-memory list, and each survivor's
// rank inside its bin counted against its bin's members (key, then index,
// descending). The cost inside a bin grows with the square of its size,
// which stays small unless very many survivors share one bin.
#pragma once

#include "row_select.h"

namespace tkp {

struct SampleArgs {
  const float* q;  // [B, ld_q] fp32, or NULL (None mode)
  int64_t ld_q;    // row stride of q in elements
  float eps;
  int32_t* sel;    // [B] selected original index (-1: survivors exceed the ranking capacity)
};

__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, RowSmem& sm) {
  v = wave_reduce_u64(v, 0ull, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
  const int l = threadIdx.x & (kWave - 1);
  if (l == 0) sm.redu[threadIdx.x / kWave] = v;
  lds_barrier();
  const uint64_t r =
      wave_reduce_u64(l < kWaves ? sm.redu[l] : 0ull, 0ull, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
  lds_barrier();
  return r;
}

// The QSample pick among the survivors of `src` ((key, idx) >= (K, I)), all
// of whose keys lie in [K, kmax]; `list` holds at least as many u64 entries
// as there are survivors. Returns the winner's original index (uniform).
// Every thread of the block must call it; the histograms are left zeroed.
template <class DT, class Src>
__device__ __forceinline__ int32_t qsample_pick(const Src& src, uint32_t K, uint32_t I, uint32_t kmax, float m,
                                                const float* __restrict__ qrow, float eps, SelSmem& ss,
                                                uint64_t* list, RowSmem& sm) {
  constexpr float kLog2e = 1.4426950408889634f;
  const int shift = shift_for_range(kmax - K);
  auto survives = [&](uint32_t key, int idx) { return key > K || (key == K && static_cast<uint32_t>(idx) >= I); };
  // 1. survivors per bin
  src.for_each([&](auto raw, int idx) {
    const uint32_t key = DT::key(raw);
    if (survives(key, idx)) atomicAdd(&ss.cnt[(key - K) >> shift], 1u);
  });
  lds_barrier();
  // 2. bin bases counted from the top: thread t owns bin kBins - 1 - t
  const int bin_t = kBins - 1 - static_cast<int>(threadIdx.x);
  const uint32_t c_t = ss.cnt[bin_t];
  const uint32_t incl = block_incl_scan_u32(c_t, ss.wtot32);
  ss.cnt[bin_t] = incl - c_t;
  lds_barrier();
  // 3. survivors placed by bin (order inside a bin is arbitrary); kmx counts the bin's members
  src.for_each([&](auto raw, int idx) {
    const uint32_t key = DT::key(raw);
    if (survives(key, idx)) {
      const uint32_t bin = (key - K) >> shift;
      const uint32_t slot = ss.cnt[bin] + atomicAdd(&ss.kmx[bin], 1u);
      list[slot] = (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(idx);
    }
  });
  lds_barrier();
  // 4. rank = bin base + members of the bin above this survivor; score; pick
  uint64_t best = 0;  // (monotone key of the score) << 32 | ~rank: the first maximum wins
  src.for_each([&](auto raw, int idx) {
    const uint32_t key = DT::key(raw);
    if (survives(key, idx)) {
      const uint32_t bin = (key - K) >> shift;
      const uint32_t lo = ss.cnt[bin], nb = ss.kmx[bin];
      const uint64_t me = (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(idx);
      uint32_t above = 0;
      for (uint32_t j = 0; j < nb; ++j) above += list[lo + j] > me ? 1u : 0u;
      const uint32_t rank = lo + above;
      const float e = __builtin_amdgcn_exp2f((DT::value(raw) - m) * kLog2e);
      const float score = e / (qrow[rank] + eps);
      const uint64_t packed = (static_cast<uint64_t>(F32T::key(__float_as_uint(score))) << 32) | (~rank);
      best = packed > best ? packed : best;
    }
  });
  best = block_max_u64(best, sm);
  const uint32_t win_rank = ~static_cast<uint32_t>(best);
  // the winner's index: the list entry at its rank is not known (order inside
  // a bin is arbitrary), so the survivor holding that rank publishes it
  src.for_each([&](auto raw, int idx) {
    const uint32_t key = DT::key(raw);
    if (survives(key, idx)) {
      const uint32_t bin = (key - K) >> shift;
      const uint32_t lo = ss.cnt[bin], nb = ss.kmx[bin];
      if (win_rank >= lo && win_rank < lo + nb) {
        const uint64_t me = (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(idx);
        uint32_t above = 0;
        for (uint32_t j = 0; j < nb; ++j) above += list[lo + j] > me ? 1u : 0u;
        if (lo + above == win_rank) ss.run_res = static_cast<uint32_t>(idx);
      }
    }
  });
  lds_barrier();
  const int32_t win = static_cast<int32_t>(ss.run_res);
  // leave the histograms zeroed for later selections
  ss.cnt[threadIdx.x] = 0;
  ss.kmx[threadIdx.x] = 0;
  lds_barrier();
  return win;
}

}  // namespace tkp
