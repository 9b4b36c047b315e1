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

#include "launch.h"
#include "row_select.h"

namespace tkp {


__device__ __forceinline__ bool wants_survivors(const SampleArgs& sa) { return sa.indices != nullptr; }

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

// Ranks of the survivors of `src` ((key, idx) >= (K, I), keys in [K, kmax])
// in descending (key, index) order: f(raw, idx, rank) for every survivor,
// once. `list` holds at least as many u64 entries as there are survivors.
// Returns the survivor count. Every thread of the block must call it; the
// histograms are left zeroed, unless kLast (the block's last use of them:
// the next row's block clears them when it starts).
template <class DT, bool kLast = false, class Src, class F>
__device__ __forceinline__ uint32_t for_each_ranked_survivor(const Src& src, uint32_t K, uint32_t I, uint32_t kmax,
                                                             SelSmem& ss, uint64_t* list, F&& f) {
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
  if (threadIdx.x == kThreads - 1) ss.bcnt = incl;  // the survivor count
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
  // 4. rank = bin base + members of the bin above this survivor
  src.for_each([&](auto raw, int idx) {
    const uint32_t key = DT::key(raw);
    if (survives(key, idx)) {
      const uint32_t bin = (key - K) >> shift;
      const uint32_t lo = ss.cnt[bin], nb = ss.kmx[bin];
      const uint64_t me = (static_cast<uint64_t>(key) << 32) | static_cast<uint32_t>(idx);
      uint32_t above = 0;
      for (uint32_t j = 0; j < nb; ++j) above += list[lo + j] > me ? 1u : 0u;
      f(raw, idx, lo + above);
    }
  });
  const uint32_t n = ss.bcnt;
  if constexpr (!kLast) {
    lds_barrier();
    // leave the histograms zeroed for later selections
    ss.cnt[threadIdx.x] = 0;
    ss.kmx[threadIdx.x] = 0;
    lds_barrier();
  }
  return n;
}

// Survivors ranked in chunks, for any number of them: the list in shared
// memory holds kRankChunk entries, and a row may keep up to 2^20 survivors.
// Chunks are taken in descending (key, index) order. Each chunk's lowest
// entry is the want-th largest survivor below the previous chunk, found by
// the radix selection of row_select.h (the key, then the index among the
// survivors holding that key: indices are distinct, so the chunk has exactly
// want members). Its members are gathered into the list and sorted there by a
// bitonic network, descending, so the member at list position j has rank
// base + j. A row with at most kRankChunk survivors takes one chunk and no
// selection.
constexpr int kRankChunk = 4096;
static_assert((kRankChunk & (kRankChunk - 1)) == 0 && kRankChunk >= 2 * kThreads,
              "the bitonic network takes a power of two, two pairs or more per thread");

// Sorts list[0, kRankChunk) descending. Pair i (i < kRankChunk / 2) joins
// positions a and a + j, a = i with a zero bit inserted at j's bit; thread t
// takes pairs t, t + 1024, ... A stage with j <= 64 keeps the pairs of each
// wave's lanes inside 128 positions of their own, so between two such stages
// only the wave's own ordering of its shared-memory accesses is needed.
__device__ __forceinline__ void bitonic_sort_desc(uint64_t* list) {
  constexpr int kPairs = kRankChunk / 2;
  for (int k = 2; k <= kRankChunk; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < kPairs; i += kThreads) {
        const int a = ((i & ~(j - 1)) << 1) | (i & (j - 1));
        const int c = a + j;
        const uint64_t x = list[a], y = list[c];
        // blocks whose k bit is clear end descending, the others ascending;
        // the last stage (k = kRankChunk) leaves the whole list descending
        const bool desc = (a & k) == 0;
        if (desc ? (x < y) : (x > y)) {
          list[a] = y;
          list[c] = x;
        }
      }
      // the next stage: j / 2, or the first of the next k (j = k); a stage
      // whose pairs span waves must see, and be seen by, every wave
      const int jn = j > 1 ? (j >> 1) : k;
      if (j > kWave || jn > kWave) {
        lds_barrier();
      } else {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
    }
  }
  lds_barrier();
}

// Calls f(value, idx, rank) for every survivor of `src` ((key, idx) >= (K, I),
// keys in [K, kmax]) whose descending rank is below limit; n is the survivor
// count (limit <= n). `list` holds kRankChunk u64 entries of free shared
// memory. Every thread of the block must call it; the histograms stay zeroed.
template <class DT, class Src, class F>
__device__ __forceinline__ void for_each_ranked_survivor_chunked(const Src& src, uint32_t K, uint32_t I,
                                                                 uint32_t kmax, uint32_t n, uint32_t limit, int V,
                                                                 SelSmem& ss, uint64_t* list, F&& f) {
  auto survives = [K, I](uint32_t key, uint32_t idx) { return key > K || (key == K && idx >= I); };
  // the survivors not yet ranked have (key, idx) <= (hk, hidx)
  uint32_t hk = kmax, hidx = 0xFFFFFFFFu;
  uint32_t base = 0;
  while (base < limit) {  // uniform; every chunk takes at least one survivor
    const uint32_t rem = n - base;
    const uint32_t want = rem < static_cast<uint32_t>(kRankChunk) ? rem : static_cast<uint32_t>(kRankChunk);
    auto pending = [&](uint32_t key, uint32_t idx) {
      return survives(key, idx) && (key < hk || (key == hk && idx <= hidx));
    };
    // the chunk's lowest member (tk, tidx)
    uint32_t tk = K, tidx = 0;
    if (rem > static_cast<uint32_t>(kRankChunk)) {
      uint32_t r = 0;
      tk = kth_largest_key(
          src, want, K, hk, [](auto raw, int) { return DT::key(raw); },
          [&](auto raw, int idx) { return pending(DT::key(raw), static_cast<uint32_t>(idx)); }, ss, &r);
      tidx = kth_largest_key(
          src, r, 0u, static_cast<uint32_t>(V - 1), [](auto, int idx) { return static_cast<uint32_t>(idx); },
          [&](auto raw, int idx) {
            const uint32_t key = DT::key(raw);
            return key == tk && pending(key, static_cast<uint32_t>(idx));
          },
          ss);
    }
    // gather the chunk: (key, index + 1) descending is (key, index) descending,
    // and the padding (0) sorts after every member
    for (int e = threadIdx.x; e < kRankChunk; e += kThreads) list[e] = 0ull;
    if (threadIdx.x == 0) ss.run_n = 0;
    lds_barrier();
    src.for_each([&](auto raw, int idx) {
      const uint32_t key = DT::key(raw);
      const uint32_t u = static_cast<uint32_t>(idx);
      if (pending(key, u) && (key > tk || (key == tk && u >= tidx))) {
        const uint32_t at = atomicAdd(&ss.run_n, 1u);
        if (at < static_cast<uint32_t>(kRankChunk)) list[at] = (static_cast<uint64_t>(key) << 32) | (u + 1u);
      }
    });
    lds_barrier();
    bitonic_sort_desc(list);
    for (uint32_t j = threadIdx.x; j < want && base + j < limit; j += kThreads) {
      const uint64_t e = list[j];
      const uint32_t key = static_cast<uint32_t>(e >> 32);
      f(DT::value(DT::raw_of_key(key)), static_cast<int>(static_cast<uint32_t>(e) - 1u), base + j);
    }
    base += want;
    // the next chunk lies strictly below (tk, tidx)
    if (tidx > 0) {
      hk = tk;
      hidx = tidx - 1;
    } else {
      hk = tk - 1;
      hidx = 0xFFFFFFFFu;
    }
    lds_barrier();  // the list is refilled by the next chunk
  }
  if (threadIdx.x == 0) ss.run_n = 0;
  lds_barrier();
}

// The QSample pick among the survivors of `src`: the first maximum of
// exp(x - m) / (q[rank] + eps). Returns the winner's original index in
// thread 0 (the only thread that stores it); the block's last use of the
// selection histograms and of the reduction slots.
template <class DT, class Src>
__device__ __forceinline__ int32_t qsample_pick(const Src& src, uint32_t K, uint32_t I, uint32_t kmax, float m,
                                                const float* __restrict__ qrow, float eps, SelSmem& ss,
                                                uint64_t* list, RowSmem& sm) {
  constexpr float kLog2e = 1.4426950408889634f;
  uint64_t best = 0;  // (monotone key of the score) << 32 | ~rank: the first maximum wins
  uint32_t best_idx = 0;
  for_each_ranked_survivor<DT, true>(src, K, I, kmax, ss, list, [&](auto raw, int idx, uint32_t rank) {
    const float e = __builtin_amdgcn_exp2f((DT::value(raw) - m) * kLog2e);
    const float score = e / (qrow[rank] + eps);
    const uint64_t packed = (static_cast<uint64_t>(F32T::key(__float_as_uint(score))) << 32) | (~rank);
    if (packed > best) {
      best = packed;
      best_idx = static_cast<uint32_t>(idx);
    }
  });
  // each wave's best and its index through shared memory, one barrier; the
  // packed values are distinct (one rank each), so one lane holds the wave's
  const uint64_t wbest = wave_reduce_u64(best, 0ull, [](uint64_t a, uint64_t b) { return a > b ? a : b; });
  const uint64_t holder = __ballot(best == wbest);
  const int src_lane = holder != 0 ? __ffsll(static_cast<unsigned long long>(holder)) - 1 : 0;
  const uint32_t widx = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(best_idx), src_lane));
  const int l = static_cast<int>(threadIdx.x) & (kWave - 1);
  if (l == 0) {
    sm.redu[threadIdx.x / kWave] = wbest;
    sm.redw[threadIdx.x / kWave] = widx;
  }
  lds_barrier();
  uint32_t pick = 0;
  if (threadIdx.x == 0) {
    uint64_t top = 0;
    for (int w = 0; w < kWaves; ++w)
      if (sm.redu[w] > top) {
        top = sm.redu[w];
        pick = sm.redw[w];
      }
  }
  return static_cast<int32_t>(pick);
}

// Z of step 4 for the survivors' probabilities: the sum of exp(x - m) over
// the top-k survivors (key >= the k-th largest key), or over the whole row
// without top-k. `cand` holds every element with key >= lo (all top-k
// survivors when k is on); `row` is the whole row, read from global memory.
// kk_known: Kk0 is already the k-th largest key (uniform), not searched again.
template <class DT, class Cand, class Row>
__device__ __forceinline__ double survivors_z(const Cand& cand, const Row& row, const RowParams& rp, uint32_t lo,
                                              uint32_t kmax, float m, SelSmem& ss, RowSmem& sm, double* redd,
                                              bool kk_known = false, uint32_t Kk0 = 0) {
  constexpr float kLog2e = 1.4426950408889634f;
  double z = 0.0;
  if (rp.k_on) {
    const uint32_t Kk = kk_known ? Kk0
                                 : kth_largest_key(
                                       cand, rp.k, lo, kmax, [](auto raw, int) { return DT::key(raw); },
                                       [](auto, int) { return true; }, ss);
    cand.for_each([&](auto raw, int) {
      if (DT::key(raw) >= Kk) z += static_cast<double>(__builtin_amdgcn_exp2f((DT::value(raw) - m) * kLog2e));
    });
  } else {  // the whole row, 4 vector loads in flight (more spill in the fp32 kernels); elements past the row read as -inf
    row.template for_each_vec_values<2>([&](int, const float (&x)[DT::kPerVec]) {
      float zv = 0.0f;
#pragma unroll
      for (int j = 0; j < DT::kPerVec; ++j) zv += __builtin_amdgcn_exp2f((x[j] - m) * kLog2e);
      z += static_cast<double>(zv);
    });
  }
  z = wave_sum_f64(z);
  const int l = threadIdx.x & (kWave - 1);
  if (l == 0) redd[threadIdx.x / kWave] = z;
  lds_barrier();
  const double r = wave_sum_f64(l < kWaves ? redd[l] : 0.0);
  lds_barrier();
  (void)sm;
  return r;
}

// The sorted-survivors output of one row: probs[r] = exp(x - m) / Z and
// indices[r] = the original index for descending ranks r < cap, then 0 and
// -1 up to cap; counts = the survivor count. The block's last use of the
// selection histograms.
template <class DT, class Src>
__device__ __forceinline__ void emit_survivors(const Src& src, uint32_t K, uint32_t I, uint32_t kmax, float m,
                                               double Z, const SampleArgs& sa, int b, SelSmem& ss, uint64_t* list) {
  constexpr float kLog2e = 1.4426950408889634f;
  float* __restrict__ prow = sa.probs == nullptr ? nullptr : sa.probs + static_cast<size_t>(b) * sa.cap;
  int32_t* __restrict__ irow = sa.indices + static_cast<size_t>(b) * sa.cap;
  const float zinv = static_cast<float>(1.0 / Z);
  const uint32_t n = for_each_ranked_survivor<DT, true>(src, K, I, kmax, ss, list, [&](auto raw, int idx, uint32_t rank) {
    if (rank < sa.cap) {
      irow[rank] = idx;
      if (prow != nullptr) prow[rank] = __builtin_amdgcn_exp2f((DT::value(raw) - m) * kLog2e) * zinv;
    }
  });
  for (int64_t r = static_cast<int64_t>(n) + threadIdx.x; r < sa.cap; r += kThreads) {
    irow[r] = -1;
    if (prow != nullptr) prow[r] = 0.0f;
  }
  if (threadIdx.x == 0) sa.counts[b] = static_cast<int32_t>(n);
}

}  // namespace tkp
