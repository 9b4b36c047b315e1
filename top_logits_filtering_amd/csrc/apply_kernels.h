// Row filter on raw logits: the aclnn entry of the ApplyTopKTopPWithSorted
// guide (§5, §6.1), which sorts each row and then filters it. No sort is
// materialised: each row's threshold pair (K, I) comes from selection
// (row_select.h) and the output is written in the original order.
//
// One 1024-thread block owns one row, so rows never exchange data and no
// global scratch is needed. The row lives either in registers (RegTile, when
// it fits in 20 16-byte vectors per thread: 163840 fp16/bf16 or 81920 fp32
// values) or is re-read from global memory on every traversal (GlobalTile).
//
// Candidate plan (default). Typical decoding rows keep a tiny top set, so:
//  1. while the row arrives, each thread tracks the two largest maxima of
//     its 16-byte vectors and, for top-p rows without top-k, an online
//     (running-max rescaled) sum of exp(x - max); rows with k above 1536
//     (16-bit values in registers) then take the four largest from the
//     vector maxima kept in shared memory;
//  2. the whole output row is written as -inf (it does not depend on the
//     data), in portions issued between the steps below, so these stores
//     drain while the block works on in registers and shared memory only (a
//     vector load or a register spill now would wait for them: vector memory
//     operations complete in order);
//  3-4. the 2048 (or 4096) per-thread maxima are actual row elements, so
//     the k-th largest of them bounds the top-k threshold from below; for
//     top-p-only rows the bound is where the mass of those maxima, walked
//     from the top, reaches (1 - t) * Z, so every element above it carries
//     at least that mass and the top-p boundary cannot lie below it. One
//     1024-bin histogram pass gives the bound L as a bin edge;
//  5. every vector whose maximum is >= L is copied into a list in shared
//     memory (placed by wave ballots, one shared-memory atomic per wave),
//     then the elements >= L of those vectors into a list of (raw, index)
//     pairs, at most 5 per thread, which the selection keeps in registers
//     (register tiles with more candidate vectors than the vector list
//     holds list their elements straight from the registers);
//  6. the exact selection (row_select.h) runs on those candidates only: one
//     wave ranks them directly when there are at most 64; joint rows whose
//     candidate keys span fewer than 1024 values take one pass of count and
//     mass histograms; other rows take range-adaptive radix passes;
//  7. once every -inf store has completed, the survivors are written over
//     them.
// Whenever a bound cannot be formed (k > 3072, top-p mass not reached) or a
// list overflows, the block falls back to the multi-pass plan, which
// rewrites the whole row; the same thread writes the same addresses in the
// same order, so the earlier -inf stores are overwritten.
//
// Multi-pass plan: the selection of row_select.h over every element of the
// row, re-read from global memory on each traversal, then one coalesced
// write. Only the candidate plan's traversals run over the register tile,
// which keeps the unrolled code small.

#pragma once

#include "launch.h"
#include "reg_tile.h"
#include "row_select.h"
#include "sample.h"

namespace tkp {

// Largest vector maxima kept per thread for the bound: two, or four for rows
// with k above kTop4From (taken after the row's arrival from the vector
// maxima in shared memory, so the arrival of other rows pays nothing). A
// bound from the k-th largest of them keeps the candidates within the list
// for k up to about three quarters of the maxima taken; beyond that a row
// goes to the multi-pass plan.
constexpr int kTopPerThread = 4;
constexpr int kTopN = kTopPerThread * kThreads;
constexpr int kTop2N = 2 * kThreads;
constexpr uint32_t kTop4From = 3 * kThreads / 2;
constexpr uint32_t kBoundMaxK2 = kTop2N;     // with two maxima per thread
constexpr uint32_t kBoundMaxK4 = 3 * kThreads;  // with four

// The first kPer of each thread's kept maxima, as a source for the bound
// passes (row_select.h); index unused (reads as 0).
template <class DT, int kPer>
struct TopMaxima {
  using raw_t = typename DT::raw_t;
  const uint32_t* top;
  template <class F>
  __device__ __forceinline__ void for_each(F&& f) const {
#pragma unroll
    for (int r = 0; r < kPer; ++r) f(static_cast<raw_t>(top[r * kThreads + threadIdx.x]), 0);
  }
};
constexpr int kMaxVecs = 20;
constexpr int kCandVecCap = 2048;  // candidate vectors kept in shared memory
constexpr int kStreamVmSlots = 32;  // streamed rows: vector maxima kept for this many layers
constexpr int kCandPerThread = 5;
// streamed rows: flags on a listed candidate's start (< 2^20) when its
// thread kept the vector in shared memory, and in which of its two entries
constexpr uint32_t kCe0Listed = 0x80000000u;
constexpr uint32_t kCe0Second = 0x40000000u;
constexpr int kRegFallbackVecs = 4;  // register tiles of up to this many vectors run the fallback in registers
constexpr int kCandCap = kCandPerThread * kThreads;  // candidate elements kept in shared memory

// When the -inf stores of a register tile are issued, as cumulative shares (in
// percent) of its vector slots: while the row arrives, then before the row
// statistics, the bound, the compaction and the selection. A wave cannot run
// ahead of its stores once the memory pipeline is full, so the stores are
// spread over the steps that follow the loads instead of issued at once;
// they then drain while those steps run.
constexpr int kStoreShare[5] = {0, 0, 20, 60, 100};
template <int NV, int STAGE>
constexpr int store_upto() {
  return (NV * kStoreShare[STAGE] + 99) / 100;
}

// (raw, index) items held in shared memory; index unused (reads as 0).
template <class DT>
struct LdsValues {
  using raw_t = typename DT::raw_t;
  const uint32_t* raw;
  int n;
  template <class F>
  __device__ __forceinline__ void for_each(F&& f) const {
    for (int c = threadIdx.x; c < n; c += kThreads) f(static_cast<raw_t>(raw[c]), 0);
  }
};

struct ApplySmem {
  RowSmem row;
  SelSmem sel;
  double redd[kWaves];
  uint32_t topm[kTopN];  // rank r of thread t's kept vector maxima at r * kThreads + t
  float run[kThreads];  // per-thread running max and rescaled exp sum (top-p-only rows)
  float acc[kThreads];
  union alignas(16) {
    uint32_t vmw[(kMaxVecs + 1) / 2][kThreads];  // per-vector maxima (16-bit bounds, two per word), steps 1-5
    uint16_t vmh[kStreamVmSlots][kThreads];      // the same for streamed rows, one per layer
    struct {
      uint32_t raw[kCandCap];  // candidate elements: raw bits
      uint32_t idx[kCandCap];  // and row indices
    } cel;                     // steps 5-7
  };
  static_assert(sizeof(cel) <= sizeof(vmh), "the candidate list shares the streamed rows' maxima memory");
  vec_t cvec[kCandVecCap];  // candidate vectors
  uint32_t ce0[kCandVecCap];
  uint32_t nvec;   // candidate vectors reserved so far
  uint32_t ncand;  // candidate elements reserved so far
  uint32_t sK, sI, sFallback;  // result of the one-wave selection
};


// The candidate elements (every element >= the bound of the row), read once
// from shared memory into registers: element c of the list goes to thread
// c % 1024, slot c / 1024.
template <class DT>
struct CandElems {
  using raw_t = typename DT::raw_t;
  uint32_t raw[kCandPerThread];
  uint32_t idx[kCandPerThread];
  int n;
  __device__ __forceinline__ void load(const ApplySmem& S, int count) {
    n = count;
#pragma unroll
    for (int s = 0; s < kCandPerThread; ++s) {
      const int c = s * kThreads + static_cast<int>(threadIdx.x);
      raw[s] = 0u;
      idx[s] = 0u;
      if (s * kThreads < n && c < n) {  // (the first test is uniform: empty slots cost nothing)
        raw[s] = S.cel.raw[c];
        idx[s] = S.cel.idx[c];
      }
    }
  }
  template <class F>
  __device__ __forceinline__ void for_each(F&& f) const {
#pragma unroll
    for (int s = 0; s < kCandPerThread; ++s) {
      if (s * kThreads < n) {  // uniform
        if (s * kThreads + static_cast<int>(threadIdx.x) < n) f(static_cast<raw_t>(raw[s]), static_cast<int>(idx[s]));
      }
    }
  }
};

__device__ __forceinline__ double block_sum_f64(double v, double* red) {
  v = wave_sum_f64(v);
  const int l = threadIdx.x & (kWave - 1);
  if (l == 0) red[threadIdx.x / kWave] = v;
  lds_barrier();
  const double r = wave_sum_f64(l < kWaves ? red[l] : 0.0);
  lds_barrier();
  return r;
}

// Multi-pass plan over any tile, then one write of the whole row (when wr).
template <class DT, class Tile>
__device__ __forceinline__ void filter_multipass(const Tile& tile, const RowParams& rp, int V, ApplySmem& S,
                                                 typename DT::raw_t* __restrict__ orow, bool wr, uint32_t& K,
                                                 uint32_t& I, const RowKnown& known = RowKnown{}) {
  using raw_t = typename DT::raw_t;
  lds_barrier();  // histograms cleared (sel_reset) before the first pass
  solve_row<DT>(tile, rp, V, S.row, S.sel, K, I, known);
  if (wr) {
    tile.store(orow, [K, I](raw_t r, int idx) {
      const uint32_t key = DT::key(r);
      return (key > K || (key == K && static_cast<uint32_t>(idx) >= I)) ? r : DT::kNegInf;
    });
  }
}

// Sampling for a row whose survivors ((key, idx) >= (K, I)) are not in a
// candidate list: None mode from the row's top position; QSample and the
// sorted survivors rank the survivors in chunks (sample.h), any number of
// them, re-reading the row on each pass.
template <class DT, class Tile>
__device__ __forceinline__ void sample_general(const Tile& tile, uint32_t K, uint32_t I, const RowParams& rp,
                                               ApplySmem& S, const SampleArgs& sa, int b, int V) {
  constexpr float kLog2e = 1.4426950408889634f;
  RowSmem& sm = S.row;
  if (sa.q == nullptr && !wants_survivors(sa)) {
    uint32_t Kt, It;
    top_position<DT>(tile, sm, Kt, It);
    if (threadIdx.x == 0 && sa.sel != nullptr) sa.sel[b] = static_cast<int32_t>(It);
    return;
  }
  float mloc = -INFINITY;
  uint32_t n = 0;
  tile.for_each([&](auto raw, int idx) {
    const uint32_t key = DT::key(raw);
    mloc = fmaxf(mloc, DT::value(raw));
    n += (key > K || (key == K && static_cast<uint32_t>(idx) >= I)) ? 1u : 0u;
  });
  const float m = block_max_f32(mloc, sm);
  n = block_sum_u32(n, sm);
  const uint32_t kmax = DT::key(DT::raw_of_value(m));
  uint64_t* list = reinterpret_cast<uint64_t*>(S.cel.raw);
  if (wants_survivors(sa)) {
    const double Z = survivors_z<DT>(tile, tile, rp, 0u, kmax, m, S.sel, sm, S.redd);
    const float zinv = static_cast<float>(1.0 / Z);
    int32_t* __restrict__ irow = sa.indices + static_cast<size_t>(b) * sa.cap;
    float* __restrict__ prow = sa.probs == nullptr ? nullptr : sa.probs + static_cast<size_t>(b) * sa.cap;
    const uint32_t limit = static_cast<int64_t>(n) < sa.cap ? n : static_cast<uint32_t>(sa.cap);
    for_each_ranked_survivor_chunked<DT>(tile, K, I, kmax, n, limit, V, S.sel, list,
                                         [&](float x, int idx, uint32_t rank) {
                                           irow[rank] = idx;
                                           if (prow != nullptr) prow[rank] = __builtin_amdgcn_exp2f((x - m) * kLog2e) * zinv;
                                         });
    for (int64_t r = static_cast<int64_t>(n) + threadIdx.x; r < sa.cap; r += kThreads) {
      irow[r] = -1;
      if (prow != nullptr) prow[r] = 0.0f;
    }
    if (threadIdx.x == 0) sa.counts[b] = static_cast<int32_t>(n);
    return;
  }
  // QSample: the first maximum of exp(x - m) / (q[rank] + eps), as qsample_pick
  const float* __restrict__ qrow = sa.q + static_cast<size_t>(b) * sa.ld_q;
  uint64_t best = 0;  // (monotone key of the score) << 32 | ~rank
  uint32_t best_idx = 0;
  for_each_ranked_survivor_chunked<DT>(tile, K, I, kmax, n, n, V, S.sel, list, [&](float x, int idx, uint32_t rank) {
    const float score = __builtin_amdgcn_exp2f((x - m) * kLog2e) / (qrow[rank] + sa.eps);
    const uint64_t packed = (static_cast<uint64_t>(F32T::key(__float_as_uint(score))) << 32) | (~rank);
    if (packed > best) {
      best = packed;
      best_idx = static_cast<uint32_t>(idx);
    }
  });
  const uint64_t win = block_max_u64(best, sm);
  if (best == win) S.sel.run_res = best_idx;  // exactly one survivor holds the winning rank
  lds_barrier();
  if (threadIdx.x == 0 && sa.sel != nullptr) sa.sel[b] = static_cast<int32_t>(S.sel.run_res);
}

// Selection among at most one wave's worth of candidates (lane j of wave 0
// holds candidate j): each candidate's rank in the descending (key, index)
// order, which is the stable ascending order read from the top, and the
// fixed-point mass strictly above it come from one sweep over the others,
// read as broadcasts from a table in shared memory (8 entries per round, so
// their reads overlap); the survivors are then a prefix of that order and
// (K, I) is the key and index of the last one. Decisions match the histogram
// selection exactly: the same masses and sums, in the same integer
// arithmetic. Wave 0 only; `tab` (64 entries) is free shared memory; the
// caller publishes the result.
template <class DT>
__device__ __forceinline__ void select_small(const ApplySmem& S, vec_t* tab, int n, const RowParams& rp, float m,
                                             uint64_t thr_ponly, bool top_only, uint32_t& K, uint32_t& I,
                                             bool& fallback) {
  fallback = n == 0;  // never: the row maximum is always a candidate
  if (fallback) return;
  const int j = static_cast<int>(threadIdx.x);
  const bool has = j < n;
  const uint32_t raw = has ? S.cel.raw[j] : 0u;
  const uint32_t idx = has ? S.cel.idx[j] : 0u;
  const uint32_t key = has ? DT::key(static_cast<typename DT::raw_t>(raw)) : 0u;
  const uint64_t comp = has ? (static_cast<uint64_t>(key) << 32 | idx) : 0ull;
  const uint64_t mass = has ? mass_fx(DT::value(static_cast<typename DT::raw_t>(raw)), m) : 0ull;
  if (has) tab[j] = vec_t{static_cast<uint32_t>(comp), static_cast<uint32_t>(comp >> 32), static_cast<uint32_t>(mass),
                          static_cast<uint32_t>(mass >> 32)};
  // one wave: its shared-memory accesses complete in order
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  uint32_t rank = 0;
  uint64_t above = 0;
  auto visit = [&](const vec_t& e) {
    const uint64_t ci = static_cast<uint64_t>(e.y) << 32 | e.x;
    if (ci > comp) {
      ++rank;
      above += static_cast<uint64_t>(e.w) << 32 | e.z;
    }
  };
  constexpr int kRound = 8;
  int i = 0;
  for (; i + kRound <= n; i += kRound) {
    vec_t e[kRound];
#pragma unroll
    for (int u = 0; u < kRound; ++u) e[u] = tab[i + u];
#pragma unroll
    for (int u = 0; u < kRound; ++u) visit(e[u]);
  }
  for (; i < n; ++i) visit(tab[i]);
  uint32_t Kk = 0;
  if (rp.k_on) {
    const uint64_t at = __ballot(has && rank == rp.k - 1);
    if (at == 0) {  // fewer than k candidates: cannot happen with a valid bound
      fallback = true;
      return;
    }
    Kk = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(key), __ffsll(static_cast<unsigned long long>(at)) - 1));
  }
  bool surv;
  if (top_only || rp.pmode == kPTopOnly) {
    surv = has && rank == 0;
  } else if (rp.pmode == kPNone) {
    K = Kk;
    I = 0;
    return;
  } else if (rp.k_on) {
    const uint64_t Z = wave_sum_u64(has && key >= Kk ? mass : 0ull);
    const uint64_t thr2 = topp_threshold(rp.t, Z);
    surv = has && (thr2 == 0 ? rank == 0 : (key >= Kk && above < thr2));
  } else {
    const uint64_t A = wave_sum_u64(mass);
    if (A < thr_ponly) {  // the boundary lies below the candidates
      fallback = true;
      return;
    }
    surv = has && above < thr_ponly;
  }
  const uint64_t last = wave_reduce_u64(surv ? comp : ~0ull, ~0ull,
                                        [](uint64_t a, uint64_t b) { return a < b ? a : b; });
  K = static_cast<uint32_t>(last >> 32);
  I = static_cast<uint32_t>(last);
}

// The candidate plan (steps 1-7 above) for a row with something to filter.
// Returns true when the row fell back to the multi-pass plan over the row in
// global memory, whose survivors the sampling stage then takes from there;
// otherwise the plan has done the sampling stage itself. K, I: the result.
template <class DT, bool kSample, class Tile, class GT>
__device__ __forceinline__ bool candidate_plan(const Tile& tile, const GT& gt, int V, const RowParams& rp,
                                               ApplySmem& S, typename DT::raw_t* __restrict__ orow, bool wr,
                                               const SampleArgs& sa, int b, uint32_t& K, uint32_t& I) {
  using raw_t = typename DT::raw_t;
  constexpr int kPV = DT::kPerVec;
  RowSmem& sm = S.row;
  SelSmem& ss = S.sel;
  // 1. per-thread statistics
  const bool ponly = rp.pmode == kPBoundary && !rp.k_on;
  constexpr float kLog2e = 1.4426950408889634f;
  float M1 = -INFINITY, M2 = -INFINITY;  // two largest vector maxima of this thread
  // rows with k above kTop4From take the four largest of the thread's vector
  // maxima once they are all in shared memory (exact there for 16-bit values)
  const bool top4 = Tile::kRegisters && sizeof(raw_t) == 2 && rp.k_on && rp.k > kTop4From;
  float run = -INFINITY, acc = 0.0f;     // acc = sum of exp(x - run), top-p-only rows
  // 16-bit upper bounds of each register vector's maximum go to shared
  // memory, two per word, so the compaction below need not revisit the data
  uint32_t vm_even = 0;
  // streamed rows: the thread's two vectors of largest maximum are kept in
  // shared memory (candidate list entries 2*tid and 2*tid+1, unused until the
  // compaction), so the compaction need not fetch them again; they hold most
  // of a row's candidates. keep_l0/keep_l1: layer held by each entry;
  // keep_top: the entry holding the largest
  int keep_l0 = -1, keep_l1 = -1, keep_top = 0;
  tile.for_each_vec_values([&](int i, const float (&x)[kPV]) {
    // the -inf store of this slot goes out as soon as its data is in (the
    // output does not depend on it): stores then drain alongside the loads
    // still in flight, and waits for later loads do not wait for them
    if constexpr (Tile::kRegisters) {
      if (wr && i < store_upto<Tile::kVecs, 0>()) tile.store_const_slot(orow, i, DT::kNegInf);
    }
    float vm = x[0];
#pragma unroll
    for (int j = 1; j < kPV; ++j) vm = fmaxf(vm, x[j]);
    if constexpr (Tile::kRegisters) {
      const uint32_t h = DT::ub16(vm);
      if ((i & 1) == 0) {
        vm_even = h;
        if (i == Tile::kVecs - 1) S.vmw[i >> 1][threadIdx.x] = h;
      } else {
        S.vmw[i >> 1][threadIdx.x] = vm_even | (h << 16);
      }
    } else {
      if (i < kStreamVmSlots) S.vmh[i][threadIdx.x] = static_cast<uint16_t>(DT::ub16(vm));
      // the new vector replaces the second largest kept one (lanes past the
      // row end hold -inf here and are never compacted)
      if (vm > M2) {
        vec_t q;
#pragma unroll
        for (int j = 0; j < kPV; ++j) set_lane<raw_t>(q, j, DT::raw_of_value(x[j]));
        const int slot = keep_top ^ 1;
        S.cvec[2 * threadIdx.x + slot] = q;
        if (slot == 0)
          keep_l0 = i;
        else
          keep_l1 = i;
        if (vm > M1) keep_top = slot;
      }
    }
    M2 = fmaxf(M2, fminf(M1, vm));
    M1 = fmaxf(M1, vm);
    if (ponly) {
      const float rn = fmaxf(run, vm);
      if (rn > -INFINITY) {
        const float scale = (run > -INFINITY) ? __builtin_amdgcn_exp2f((run - rn) * kLog2e) : 0.0f;
        float e[kPV];
#pragma unroll
        for (int j = 0; j < kPV; ++j) e[j] = __builtin_amdgcn_exp2f((x[j] - rn) * kLog2e);
#pragma unroll
        for (int w = kPV / 2; w > 0; w >>= 1)
#pragma unroll
          for (int j = 0; j < w; ++j) e[j] += e[j + w];
        acc = acc * scale + e[0];
        run = rn;
      }
    }
  });

  // The per-thread statistics go to shared memory, so no vector register
  // holds them across the stores below.
  S.topm[threadIdx.x] = DT::raw_of_value(M1);
  S.topm[kThreads + threadIdx.x] = DT::raw_of_value(M2);
  if constexpr (Tile::kRegisters && sizeof(raw_t) == 2) {
    if (top4) {  // uniform
      float a[kTopPerThread];
#pragma unroll
      for (int r = 0; r < kTopPerThread; ++r) a[r] = -INFINITY;
#pragma unroll
      for (int i = 0; i < Tile::kVecs; ++i) {  // this thread's own entries: no barrier needed
        float v = DT::ub16_value((S.vmw[i >> 1][threadIdx.x] >> ((i & 1) * 16)) & 0xFFFFu);
#pragma unroll
        for (int r = 0; r < kTopPerThread; ++r) {
          const float t = fmaxf(a[r], v);
          v = fminf(a[r], v);
          a[r] = t;
        }
      }
#pragma unroll
      for (int r = 0; r < kTopPerThread; ++r) S.topm[r * kThreads + threadIdx.x] = DT::raw_of_value(a[r]);
    }
  }
  S.run[threadIdx.x] = run;
  S.acc[threadIdx.x] = acc;

  if (threadIdx.x == 0) {  // read after the barriers of step 3
    S.nvec = 0;
    S.ncand = 0;
  }

  // 2. the whole row as -inf, in portions issued from here on (register
  // tiles) or at once after the compaction, whose reads of candidate vectors
  // would otherwise wait behind the stores (streamed rows). From here until
  // the survivors are written a register tile's block touches only registers
  // and shared memory, so nothing waits behind these stores while they drain.
  if constexpr (Tile::kRegisters)
    if (wr) tile.template store_const_range<store_upto<Tile::kVecs, 0>(), store_upto<Tile::kVecs, 1>()>(orow, DT::kNegInf);
  // 3. row maximum, smallest finite per-thread maximum, Z for top-p-only rows
  const float M1s = DT::value(static_cast<raw_t>(S.topm[threadIdx.x]));
  uint32_t klo = 0xFFFFFFFFu;  // smallest key among finite maxima (each thread's come in descending order)
#pragma unroll
  for (int r = 0; r < kTopPerThread; ++r) {
    if (r < 2 || top4) {  // uniform
      const float Mr = DT::value(static_cast<raw_t>(S.topm[r * kThreads + threadIdx.x]));
      if (Mr > -INFINITY) klo = DT::key(DT::raw_of_value(Mr));
    }
  }
  float m;
  block_max_f32_min_u32(M1s, klo, sm, m, klo);
  const uint32_t kmax = DT::key(DT::raw_of_value(m));
  uint64_t thr = 0;
  double z_row = 0.0;  // top-p-only rows: sum of exp(x - m) over the whole row
  if (ponly) {
    const float r = S.run[threadIdx.x];
    const double zt = (r > -INFINITY) ? static_cast<double>(S.acc[threadIdx.x]) *
                                            static_cast<double>(__builtin_amdgcn_exp2f((r - m) * kLog2e))
                                      : 0.0;
    z_row = block_sum_f64(zt, S.redd);  // >= 1: the maximum contributes exp(0)
    thr = topp_threshold(rp.t, static_cast<uint64_t>(z_row * 8796093022208.0));  // Z * 2^43
  }

  if constexpr (Tile::kRegisters)
    if (wr) tile.template store_const_range<store_upto<Tile::kVecs, 1>(), store_upto<Tile::kVecs, 2>()>(orow, DT::kNegInf);
  // 4. candidate bound L
  const TopMaxima<DT, 2> top2{S.topm};
  const bool top_only = rp.pmode == kPTopOnly || (ponly && thr == 0);
  // min-p alone: its survivors lie above m + ln(min_p), so that floor bounds them
  const bool mp_only = rp.mp_on && !rp.k_on && rp.pmode == kPNone;
  uint32_t L = kmax;
  bool fast = klo <= kmax;
  auto key_of = [](auto raw, int) { return DT::key(raw); };
  if (rp.k_on) {
    if (top4)
      fast = fast && rp.k <= kBoundMaxK4 &&
             kth_largest_bound(TopMaxima<DT, kTopPerThread>{S.topm}, rp.k, klo, kmax, key_of, ss, L);
    else
      fast = fast && rp.k <= kBoundMaxK2 && kth_largest_bound(top2, rp.k, klo, kmax, key_of, ss, L);
  } else if (mp_only) {
    L = key_floor<DT>(min_p_floor(m, rp.minp));
  } else if (!top_only) {
    fast = fast && topp_bound<DT>(top2, klo, kmax, m, thr, ss, L);
  }
  // Fallbacks are taken at the very end, after the candidate plan's code:
  // keeping the multi-pass plan's global loads out of the paths above keeps
  // the compiler from waiting on the -inf stores before they are needed.
  bool fallback = !fast;

  if constexpr (Tile::kRegisters)
    if (wr) tile.template store_const_range<store_upto<Tile::kVecs, 2>(), store_upto<Tile::kVecs, 3>()>(orow, DT::kNegInf);
  // 5. candidates: every vector whose maximum is >= L is packed into a list
  // in shared memory (placed by wave ballots); then the elements >= L of
  // those vectors are packed into a second list (raw bits and row index),
  // each thread taking one or two listed vectors. The list orders do not
  // matter: every statistic taken below is order-independent, and ties are
  // resolved by the stored indices.
  const float Lf = DT::value(DT::raw_of_key(L));
  // streamed rows: the layers' vector maxima are in shared memory when they fit
  const bool vm_in_lds = !Tile::kRegisters && V <= kStreamVmSlots * kThreads * kPV;
  uint32_t nvec = 0;
  int ncand = 0;
  if (!fallback) {
    auto is_cand = [&](int i, int e0) {
      float vmv;
      if constexpr (Tile::kRegisters) {
        vmv = DT::ub16_value((S.vmw[i >> 1][threadIdx.x] >> ((i & 1) * 16)) & 0xFFFFu);
      } else {
        const vec_t q = tile.vec_at(i, e0);
        vmv = -INFINITY;
  #pragma unroll
        for (int j = 0; j < kPV; ++j)
          if (e0 + j < V) vmv = fmaxf(vmv, DT::value(lane_of<raw_t>(q, j)));
      }
      return vmv >= Lf;
    };
    if constexpr (Tile::kRegisters) {
      // one pass over the register slots: each slot's ballot is kept (uniform,
      // so in scalar registers); one shared-memory atomic per wave reserves the
      // wave's run of the list
      uint64_t masks[Tile::kVecs];
      uint32_t wtotal = 0;
      tile.for_each_slot([&](int i, int e0) {
        masks[i] = __ballot(is_cand(i, e0));
        wtotal += static_cast<uint32_t>(__popcll(masks[i]));
      });
      uint32_t pos0 = 0;
      if ((threadIdx.x & (kWave - 1)) == 0) pos0 = atomicAdd(&S.nvec, wtotal);
      pos0 = __builtin_amdgcn_readfirstlane(pos0);
      const uint32_t lane = threadIdx.x & (kWave - 1);
      tile.for_each_slot([&](int i, int e0) {
        if (masks[i] != 0) {  // uniform: slots without candidates in this wave cost nothing
          // the lane's bit of the ballot (no second shared-memory read, whose
          // latency would be paid once per slot)
          if ((masks[i] >> lane) & 1ull) {
            const uint32_t pos = pos0 + lanes_below(masks[i]);
            if (pos < static_cast<uint32_t>(kCandVecCap)) {
              S.cvec[pos] = tile.vec_at(i, e0);
              S.ce0[pos] = static_cast<uint32_t>(e0);
            }
          }
          pos0 += static_cast<uint32_t>(__popcll(masks[i]));
        }
      });
    } else if (vm_in_lds) {
      // streamed rows with the layer maxima in shared memory: each thread
      // marks its candidate layers in a bit mask (the shared-memory reads
      // are issued together), reserves room for them with one shared-memory
      // atomic, and lists them
      static_assert(kStreamVmSlots <= 32, "one mask bit per layer");
      const int tid = static_cast<int>(threadIdx.x);
      // every slot is read (entries of layers past the row are not
      // meaningful and are masked out below), so no read waits on a branch
      uint32_t h[kStreamVmSlots];
#pragma unroll
      for (int i = 0; i < kStreamVmSlots; ++i) h[i] = S.vmh[i][tid];
      uint32_t mine = 0;
#pragma unroll
      for (int i = 0; i < kStreamVmSlots; ++i) {
        const bool in_row = i * Tile::kSpan + tid * kPV < V;
        mine |= static_cast<uint32_t>(in_row & (DT::ub16_value(h[i]) >= Lf)) << i;
      }
      // the wave's run of the list: a lane scan of the counts, one
      // shared-memory atomic per wave
      const uint32_t n = static_cast<uint32_t>(__popc(mine));
      const uint32_t incl = wave_incl_scan_u32(n);
      const uint32_t wtot = lane63_u32(incl);
      uint32_t base = 0;
      if (wtot != 0 && (threadIdx.x & (kWave - 1)) == 0) base = atomicAdd(&S.nvec, wtot);
      uint32_t pos = __builtin_amdgcn_readfirstlane(base) + incl - n;
      while (mine != 0) {
        const int i = __ffs(mine) - 1;
        mine &= mine - 1;
        if (pos < static_cast<uint32_t>(kCandVecCap)) {
          // a kept vector is flagged with its entry, instead of being fetched again
          const uint32_t kept = i == keep_l0 ? kCe0Listed : i == keep_l1 ? kCe0Listed | kCe0Second : 0u;
          S.ce0[pos] = static_cast<uint32_t>(i * Tile::kSpan + tid * kPV) | kept;
        }
        ++pos;
      }
    } else {
      // streamed rows: one atomic per wave for each slot holding candidates
      tile.for_each_slot([&](int i, int e0) {
        const bool c = is_cand(i, e0);
        const uint64_t mask = __ballot(c);
        if (mask != 0) {
          uint32_t pos0 = 0;
          if ((threadIdx.x & (kWave - 1)) == 0) pos0 = atomicAdd(&S.nvec, static_cast<uint32_t>(__popcll(mask)));
          pos0 = __builtin_amdgcn_readfirstlane(pos0);
          if (c) {  // only the position: the vectors are gathered together below
            const uint32_t pos = pos0 + lanes_below(mask);
            if (pos < static_cast<uint32_t>(kCandVecCap)) S.ce0[pos] = static_cast<uint32_t>(e0);
          }
        }
      });
    }
    lds_barrier();
    nvec = S.nvec;
    fallback = nvec > static_cast<uint32_t>(kCandVecCap);
    bool listed = false;  // the elements are already in the candidate list
    if constexpr (Tile::kRegisters) {
      if (fallback) {  // uniform
        // more candidate vectors than their list holds (large k, wide rows):
        // each thread counts its elements >= L in its candidate slots, a
        // block scan places them, and each thread writes its own. The slot
        // mask is taken first: the element list overwrites the maxima.
        uint32_t slots = 0;
        uint32_t mine = 0;
        tile.for_each_vec([&](int i, const vec_t& q, int e0) {
          if (is_cand(i, e0)) {
            slots |= 1u << i;
#pragma unroll
            for (int j = 0; j < kPV; ++j)
              mine += (e0 + j < V && DT::value(lane_of<raw_t>(q, j)) >= Lf) ? 1u : 0u;
          }
        });
        const uint32_t incl = block_incl_scan_u32(mine, ss.wtot32);
        if (threadIdx.x == kThreads - 1) S.ncand = incl;
        lds_barrier();  // every slot mask is taken before the list is written
        uint32_t at = incl - mine;
        tile.for_each_vec([&](int i, const vec_t& q, int e0) {
          if ((slots >> i) & 1u) {
#pragma unroll
            for (int j = 0; j < kPV; ++j) {
              const raw_t r = lane_of<raw_t>(q, j);
              if (e0 + j < V && DT::value(r) >= Lf) {
                if (at < static_cast<uint32_t>(kCandCap)) {
                  S.cel.raw[at] = r;
                  S.cel.idx[at] = static_cast<uint32_t>(e0 + j);
                }
                ++at;
              }
            }
          }
        });
        lds_barrier();
        ncand = static_cast<int>(S.ncand);
        fallback = ncand > kCandCap;
        listed = true;
      }
    }
    if (!fallback && !listed) {
      // each thread takes listed vectors tid and tid + 1024 (a streamed row
      // requests both from global memory at once); per element lane j of the
      // vectors a wave ballot places the elements >= L
      constexpr int kRounds = kCandVecCap / kThreads;
      vec_t qs[kRounds];
      int e0s[kRounds];
#pragma unroll
      for (int r = 0; r < kRounds; ++r) {
        const int vi = static_cast<int>(threadIdx.x) + r * kThreads;
        qs[r] = vec_t{0u, 0u, 0u, 0u};
        e0s[r] = V;  // past the row: no element of an unused slot passes
        if (vi < static_cast<int>(nvec)) {
          const uint32_t ce = S.ce0[vi];
          e0s[r] = static_cast<int>(ce & ~(kCe0Listed | kCe0Second));
          if constexpr (Tile::kRegisters) {
            qs[r] = S.cvec[vi];
          } else if (ce & kCe0Listed) {  // kept by its thread: entry 2*owner (+1)
            const int owner = (e0s[r] % Tile::kSpan) / kPV;
            qs[r] = S.cvec[2 * owner + ((ce & kCe0Second) ? 1 : 0)];
          } else {
            qs[r] = tile.gather(e0s[r]);
          }
        }
      }
#pragma unroll
      for (int r = 0; r < kRounds; ++r) {
        if (r * kThreads >= static_cast<int>(nvec)) break;  // uniform
        const vec_t q = qs[r];
        const int e0 = e0s[r];
        uint64_t mk[kPV];
        uint32_t wtot = 0;
#pragma unroll
        for (int j = 0; j < kPV; ++j) {
          mk[j] = __ballot(e0 + j < V && DT::value(lane_of<raw_t>(q, j)) >= Lf);
          wtot += static_cast<uint32_t>(__popcll(mk[j]));
        }
        // one shared-memory atomic per wave that has elements
        uint32_t pos0 = 0;
        if (wtot != 0 && (threadIdx.x & (kWave - 1)) == 0) pos0 = atomicAdd(&S.ncand, wtot);
        uint32_t pos = __builtin_amdgcn_readfirstlane(pos0);
#pragma unroll
        for (int j = 0; j < kPV; ++j) {
          if (mk[j] != 0) {
            const raw_t r = lane_of<raw_t>(q, j);
            if (e0 + j < V && DT::value(r) >= Lf) {
              const uint32_t at = pos + lanes_below(mk[j]);
              if (at < static_cast<uint32_t>(kCandCap)) {
                S.cel.raw[at] = r;
                S.cel.idx[at] = static_cast<uint32_t>(e0 + j);
              }
            }
            pos += static_cast<uint32_t>(__popcll(mk[j]));
          }
        }
      }
      lds_barrier();
      ncand = static_cast<int>(S.ncand);
      fallback = ncand > kCandCap;
    }
  }

  // The last portion of the -inf stores. Joint rows selected in one pass
  // issue it inside the selection instead: waves 1-15 while wave 0 alone
  // scans the histograms (so that scan runs while they wait for room to
  // store), wave 0 right after.
  auto last_stores = [&]() {
    if (!wr) return;
    if constexpr (Tile::kRegisters)
      tile.template store_const_range<store_upto<Tile::kVecs, 3>(), store_upto<Tile::kVecs, 4>()>(orow, DT::kNegInf);
    else
      tile.store_const(orow, DT::kNegInf);
  };
  const bool small = !fallback && ncand <= kWave;
  const bool one_key_bins = shift_for_range(kmax - L) == 0;
  const bool joint_one_pass = !fallback && !small && rp.k_on && rp.pmode == kPBoundary && one_key_bins;
  const bool topk_one_pass = !fallback && !small && rp.k_on && rp.pmode == kPNone && one_key_bins;
  // paths with a one-wave step take the last stores inside it
  const bool shadow_stores = small || joint_one_pass || topk_one_pass;
  if (!shadow_stores && !fallback) last_stores();  // a fallback rewrites the whole row
  // 6. exact selection on the candidates (all elements with key in [L, kmax])
  CandElems<DT> cs;
  cs.load(S, fallback ? 0 : ncand);
  K = 0;
  I = 0;
  // the key of the k-th largest when a selection path below has found it
  // (the sorted survivors' Z sums the top-k survivors and need not find it again)
  uint32_t kk_sel = 0;
  bool kk_found = false;
  if (small) {
    if (threadIdx.x >= kWave) last_stores();
    if (threadIdx.x < kWave) {
      bool fb;
      // the candidate vectors' list is no longer needed: its first entries hold the table
      select_small<DT>(S, S.cvec, ncand, rp, m, thr, top_only, K, I, fb);
      if (threadIdx.x == 0) {
        S.sK = K;
        S.sI = I;
        S.sFallback = fb ? 1u : 0u;
      }
      last_stores();
    }
    lds_barrier();
    K = S.sK;
    I = S.sI;
    fallback = S.sFallback != 0;
  } else if (!fallback) {
    if (top_only && !rp.k_on) {
      top_position<DT>(cs, sm, K, I);
    } else if (topk_one_pass) {
      // the k-th largest from one count pass: every bin of [L, kmax] holds one key
      cs.for_each([&](auto raw, int) { atomicAdd(&ss.cnt[DT::key(raw) - L], 1u); });
      lds_barrier();
      if (threadIdx.x >= kWave) last_stores();
      sel_pick_count(ss, rp.k);
      if (threadIdx.x < kWave) last_stores();
      K = L + static_cast<uint32_t>(ss.bin);
      kk_sel = K;
      kk_found = true;
    } else if (joint_one_pass) {
      // top-k and top-p from one pass: every bin of [L, kmax] holds one key
      cs.for_each([&](auto raw, int) {
        const uint32_t bin = DT::key(raw) - L;
        atomicAdd(&ss.mass[bin], mass_fx(DT::value(raw), m));
        atomicAdd(&ss.cnt[bin], 1u);
      });
      lds_barrier();
      if (threadIdx.x >= kWave) last_stores();
      sel_pick_joint(ss, rp.k, rp.t);
      if (threadIdx.x < kWave) last_stores();
      const uint64_t thr2 = ss.thr;
      kk_sel = L + static_cast<uint32_t>(ss.kbin);
      kk_found = true;
      if (thr2 == 0) {
        top_position<DT>(cs, sm, K, I);
      } else {
        K = L + static_cast<uint32_t>(ss.bin);
        I = boundary_index<DT>(cs, K, thr2 - ss.above64, ss.bcnt, ss.bmass, V, ss);
      }
    } else {
      uint32_t Kk = L;
      if (rp.k_on)
        Kk = kth_largest_key(
            cs, rp.k, L, kmax, [](auto raw, int) { return DT::key(raw); }, [](auto, int) { return true; }, ss);
      kk_sel = Kk;
      kk_found = rp.k_on;
      if (rp.pmode == kPNone) {
        K = Kk;
      } else if (rp.pmode == kPTopOnly) {
        top_position<DT>(cs, sm, K, I);
      } else if (rp.k_on) {
        uint64_t z = 0;
        cs.for_each([&](auto raw, int) {
          if (DT::key(raw) >= Kk) z += mass_fx(DT::value(raw), m);
        });
        const uint64_t Z = block_sum_u64(z, sm);
        const uint64_t thr2 = topp_threshold(rp.t, Z);
        if (thr2 == 0)
          top_position<DT>(cs, sm, K, I);
        else
          topp_boundary<DT>(cs, Kk, kmax, m, thr2, V, ss, K, I);
      } else {
        uint64_t a = 0;
        cs.for_each([&](auto raw, int) { a += mass_fx(DT::value(raw), m); });
        const uint64_t A = block_sum_u64(a, sm);
        if (A < thr)  // the boundary lies below the candidates
          fallback = true;
        else
          topp_boundary<DT>(cs, L, kmax, m, thr, V, ss, K, I);
      }
    }
  }

  // min-p: the smallest candidate key that survives it; every stage keeps a
  // suffix of the stable order, so the tighter pair wins. Its threshold is
  // either above L (then a candidate holds it) or below every candidate.
  if (!fallback && rp.mp_on) combine_min_p(min_p_key<DT>(cs, m, rp.minp, sm), K, I);

  if constexpr (kSample) {
    if (!fallback && wants_survivors(sa)) {  // every survivor is a candidate
      // (top-p-only rows reuse the row sum of step 3; other rows without k
      // sum the whole row re-read from global memory: keeping the register
      // tile live through the ranking below would spill it)
      const double Z = ponly ? z_row : survivors_z<DT>(cs, gt, rp, L, kmax, m, ss, sm, S.redd, kk_found, kk_sel);
      emit_survivors<DT>(cs, K, I, kmax, m, Z, sa, b, ss, reinterpret_cast<uint64_t*>(S.cel.raw));
    } else if (!fallback) {  // every survivor is a candidate
      int32_t pick;
      if (sa.q == nullptr) {
        uint32_t Kt, It;
        top_position<DT>(cs, sm, Kt, It);
        pick = static_cast<int32_t>(It);
      } else {
        pick = qsample_pick<DT>(cs, K, I, kmax, m, sa.q + static_cast<size_t>(b) * sa.ld_q, sa.eps, ss,
                                reinterpret_cast<uint64_t*>(S.cel.raw), sm);
      }
      if (threadIdx.x == 0 && sa.sel != nullptr) sa.sel[b] = pick;
    }
  }

  // 7. survivors over the -inf row, once every -inf store has completed
  if (!fallback) {
    if (wr) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      cs.for_each([&](auto raw, int idx) {
        const uint32_t key = DT::key(raw);
        if (key > K || (key == K && static_cast<uint32_t>(idx) >= I)) orow[gt.out_at(idx)] = raw;
      });
    }
  } else if constexpr (Tile::kRegisters && Tile::kVecs <= kRegFallbackVecs) {
    // short register rows run the multi-pass plan over the registers: each
    // traversal then costs no memory latency (longer rows re-read global
    // memory, which keeps the unrolled code of their kernels small)
    filter_multipass<DT>(tile, rp, V, S, orow, wr, K, I, RowKnown{true, m, ponly ? thr : 0});
    if constexpr (kSample) sample_general<DT>(tile, K, I, rp, S, sa, b, V);
  } else {
    filter_multipass<DT>(gt, rp, V, S, orow, wr, K, I, RowKnown{true, m, ponly ? thr : 0});
    return true;
  }
  return false;
}


// `tile` holds the row (registers or global); `gt` is the same row in
// global memory, re-read by the multi-pass fallback (a GlobalTile, strided
// for views with a non-unit element stride). kSample adds the sampling stage
// (sample.h) and makes the row's output optional (wr).
template <class DT, bool kSample, class Tile, class GT>
__device__ __forceinline__ void filter_row(const Tile& tile, const GT& gt, int V, const RowParams& rp,
                                           bool use_candidates, ApplySmem& S,
                                           typename DT::raw_t* __restrict__ orow, bool wr_out,
                                           const SampleArgs& sa, int b) {
  const bool wr = kSample ? wr_out : true;
  using raw_t = typename DT::raw_t;
  constexpr int kPV = DT::kPerVec;
  RowSmem& sm = S.row;
  SelSmem& ss = S.sel;
  sel_reset(ss);

  if constexpr (kSample) {
    // argmax without the filtered row: the pick is the row's top position
    // (the maximum always survives every stage), so no selection is needed
    if (sa.q == nullptr && !wr && !wants_survivors(sa)) {
      // per thread the last vector holding its maximum (later vectors hold
      // higher indices), then the highest lane of it holding the row's
      float best = -INFINITY;
      vec_t bq = {0u, 0u, 0u, 0u};
      int be0 = -1;
      tile.for_each_vec_values([&](int i, const float (&x)[kPV]) {
        float vm = x[0];
#pragma unroll
        for (int j = 1; j < kPV; ++j) vm = fmaxf(vm, x[j]);
        if (vm >= best && vm > -INFINITY) {
          best = vm;
          bq = tile.vec_at(i, i * Tile::kSpan + static_cast<int>(threadIdx.x) * kPV);
          be0 = i * Tile::kSpan + static_cast<int>(threadIdx.x) * kPV;
        }
      });
      const float mrow = block_max_f32(best, sm);
      int idx = -1;
      if (be0 >= 0 && best == mrow) {
#pragma unroll
        for (int j = 0; j < kPV; ++j)
          if (be0 + j < V && DT::value(lane_of<raw_t>(bq, j)) == mrow) idx = be0 + j;
      }
      idx = static_cast<int>(block_max_u32(static_cast<uint32_t>(idx + 1), sm)) - 1;
      if (threadIdx.x == 0 && sa.sel != nullptr) sa.sel[b] = idx < 0 ? 0 : idx;
      return;
    }
  }
  uint32_t K = 0, I = 0;
  bool general = true;  // the survivors are (key, idx) >= (K, I) of the whole row, re-read from global memory
  if (!row_filters(rp)) {  // nothing to filter
    if (wr) tile.store(orow, [](raw_t r, int) { return r; });
  } else if (!use_candidates) {
    filter_multipass<DT>(gt, rp, V, S, orow, wr, K, I);
  } else {
    general = candidate_plan<DT, kSample>(tile, gt, V, rp, S, orow, wr, sa, b, K, I);
  }
  // one place for the general sampling path: each inlined copy of it costs
  // registers in the kernels whose row is held in registers
  if constexpr (kSample)
    if (general) sample_general<DT>(gt, K, I, rp, S, sa, b, V);
}

template <class DT, int NVEC, bool kSample>
__global__ __launch_bounds__(kThreads) void apply_regs_kernel(const typename DT::raw_t* __restrict__ logits,
                                                              const typename DT::raw_t* __restrict__ p,
                                                              const int32_t* __restrict__ k,
                                                              const typename DT::raw_t* __restrict__ min_p,
                                                              typename DT::raw_t* __restrict__ out, int V,
                                                              RowStrides ld, int use_candidates, SampleArgs sa) {
  __shared__ ApplySmem S;
  const int b = blockIdx.x;
  const size_t offx = static_cast<size_t>(b) * static_cast<size_t>(ld.x);
  const size_t offo = static_cast<size_t>(b) * static_cast<size_t>(ld.o);
  // p[b], k[b] and min_p[b] are fetched before the row and used after it is requested
  const RowParamsRaw<DT> rpr = fetch_row_params<DT>(p, k, min_p, b);
  RegTile<DT, NVEC> tile;
  tile.load(logits + offx, 0, V);
  const RowParams rp = decode_row_params<DT>(rpr, V);
  GlobalTile<DT> gt;
  gt.load(logits + offx, 0, V);
  filter_row<DT, kSample>(tile, gt, V, rp, use_candidates != 0, S, out + offo, out != nullptr, sa, b);
}

template <class DT, bool kSample>
__global__ __launch_bounds__(kThreads) void apply_stream_kernel(const typename DT::raw_t* __restrict__ logits,
                                                                const typename DT::raw_t* __restrict__ p,
                                                                const int32_t* __restrict__ k,
                                                                const typename DT::raw_t* __restrict__ min_p,
                                                                typename DT::raw_t* __restrict__ out, int V,
                                                                RowStrides ld, int use_candidates, SampleArgs sa) {
  __shared__ ApplySmem S;
  const int b = blockIdx.x;
  const size_t offx = static_cast<size_t>(b) * static_cast<size_t>(ld.x);
  const size_t offo = static_cast<size_t>(b) * static_cast<size_t>(ld.o);
  const RowParams rp = decode_row_params<DT>(p, k, min_p, b, V);
  GlobalTile<DT> tile;
  tile.load(logits + offx, 0, V);
  filter_row<DT, kSample>(tile, tile, V, rp, use_candidates != 0, S, out + offo, out != nullptr, sa, b);
}

// Views with a non-unit element stride: element (b, v) of logits sits at
// b * ld.x + v * ld.xc and of out at b * ld.o + v * ld.oc; p, k and min_p
// step by ld.pc, ld.kc and ld.mc. The streamed plan with element accesses.
template <class DT>
__global__ __launch_bounds__(kThreads) void apply_strided_kernel(const typename DT::raw_t* __restrict__ logits,
                                                                 const typename DT::raw_t* __restrict__ p,
                                                                 const int32_t* __restrict__ k,
                                                                 const typename DT::raw_t* __restrict__ min_p,
                                                                 typename DT::raw_t* __restrict__ out, int V,
                                                                 RowStrides ld, int use_candidates) {
  __shared__ ApplySmem S;
  const int b = blockIdx.x;
  const RowParams rp = decode_row_params<DT>(
      fetch_row_params_strided<DT>(p, k, min_p, static_cast<int64_t>(b), ld.pc, ld.kc, ld.mc), V);
  GlobalTile<DT, true> tile;
  tile.load_strided(logits + static_cast<size_t>(b) * static_cast<size_t>(ld.x), V, ld.xc, ld.oc);
  const SampleArgs sa{nullptr, 0, 0.0f, nullptr, nullptr, nullptr, nullptr, 0};
  filter_row<DT, false>(tile, tile, V, rp, use_candidates != 0, S, out + static_cast<size_t>(b) * static_cast<size_t>(ld.o),
                        true, sa, b);
}

template <class DT, int NVEC, bool kSample>
void launch_regs(const void* logits, const void* p, const int32_t* k, const void* min_p, void* out, int64_t B,
                 int64_t V, RowStrides ld, int use_candidates, const SampleArgs& sa, hipStream_t stream) {
  using raw_t = typename DT::raw_t;
  hipLaunchKernelGGL((apply_regs_kernel<DT, NVEC, kSample>), dim3(static_cast<unsigned>(B)), dim3(kThreads), 0,
                     stream, static_cast<const raw_t*>(logits), static_cast<const raw_t*>(p), k,
                     static_cast<const raw_t*>(min_p), static_cast<raw_t*>(out), static_cast<int>(V), ld,
                     use_candidates, sa);
}

// The argmax of streamed rows when neither the filtered row, q nor the
// survivors are asked for: the row maximum survives every stage, so the pick
// is the top position of the stable order (the highest index holding the
// maximum; -0 and +0 tie). Only a block reduction is kept in shared memory,
// so two blocks share a compute unit and one row's loads overlap another's
// reductions.
template <class DT>
__global__ __launch_bounds__(kThreads, 2) void argmax_stream_kernel(const typename DT::raw_t* __restrict__ logits,
                                                                     int V, int64_t ld_x, int32_t* __restrict__ sel) {
  __shared__ RowSmem sm;
  constexpr int kPV = DT::kPerVec;
  const int b = blockIdx.x;
  GlobalTile<DT> gt;
  gt.load(logits + static_cast<size_t>(b) * static_cast<size_t>(ld_x), 0, V);
  float best = -INFINITY;
  int bidx = -1;  // a thread's elements come in ascending index order: ">=" keeps the last maximum
  gt.template for_each_vec_values<4>([&](int i, const float (&x)[kPV]) {
    const int e0 = i * GlobalTile<DT>::kSpan + static_cast<int>(threadIdx.x) * kPV;
#pragma unroll
    for (int j = 0; j < kPV; ++j) {
      if (x[j] >= best && x[j] > -INFINITY) {
        best = x[j];
        bidx = e0 + j;
      }
    }
  });
  const float mrow = block_max_f32(best, sm);
  const int idx = (bidx >= 0 && best == mrow) ? bidx : -1;
  const int top = static_cast<int>(block_max_u32(static_cast<uint32_t>(idx + 1), sm)) - 1;
  if (threadIdx.x == 0) sel[b] = top < 0 ? 0 : top;
}

// kSample: the sampling stage (sa), and out may be NULL; otherwise sa is unused.
// Rows [0, B) in one launch of one block per row (B <= kMaxLaunchBlocks).
template <class DT, bool kSample>
hipError_t launch_apply_rows(const void* logits, const void* p, const int32_t* k, const void* min_p, void* out,
                             int64_t B, int64_t V, RowStrides ld, int policy, hipStream_t stream,
                             const SampleArgs& sa) {
  using raw_t = typename DT::raw_t;
  constexpr int span = kThreads * DT::kPerVec;
  const int64_t vecs = (V + span - 1) / span;
  const int use_candidates = policy == kPlanGeneral ? 0 : 1;
  if constexpr (!kSample) {
    if (ld.elementwise) {
      hipLaunchKernelGGL((apply_strided_kernel<DT>), dim3(static_cast<unsigned>(B)), dim3(kThreads), 0, stream,
                         static_cast<const raw_t*>(logits), static_cast<const raw_t*>(p), k,
                         static_cast<const raw_t*>(min_p), static_cast<raw_t*>(out), static_cast<int>(V), ld,
                         use_candidates);
      return hipGetLastError();
    }
  }
  // register tiles move whole 16-byte vectors: every row must start 16-byte aligned
  constexpr int64_t es = static_cast<int64_t>(sizeof(raw_t));
  const bool vec_ok = (V % DT::kPerVec) == 0 && (reinterpret_cast<uintptr_t>(logits) & 15u) == 0 &&
                      (reinterpret_cast<uintptr_t>(out) & 15u) == 0 && (ld.x * es) % 16 == 0 &&
                      (out == nullptr || (ld.o * es) % 16 == 0);
  // the sampling kernels hold at most 19 vectors per thread in registers
  // (20 would spill in fp16); longer rows are streamed
  constexpr int64_t max_vecs = kSample ? 19 : kMaxVecs;
  if (policy != kPlanAuto || vecs > max_vecs || !vec_ok) {
    if constexpr (kSample) {
      if (sa.q == nullptr && out == nullptr && sa.indices == nullptr) {
        if (sa.sel != nullptr)
          hipLaunchKernelGGL((argmax_stream_kernel<DT>), dim3(static_cast<unsigned>(B)), dim3(kThreads), 0, stream,
                             static_cast<const raw_t*>(logits), static_cast<int>(V), ld.x, sa.sel);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((apply_stream_kernel<DT, kSample>), dim3(static_cast<unsigned>(B)), dim3(kThreads), 0, stream,
                       static_cast<const raw_t*>(logits), static_cast<const raw_t*>(p), k,
                       static_cast<const raw_t*>(min_p), static_cast<raw_t*>(out), static_cast<int>(V), ld,
                       use_candidates, sa);
  } else if (vecs <= 1) {
    launch_regs<DT, 1, kSample>(logits, p, k, min_p, out, B, V, ld, use_candidates, sa, stream);
  } else if (vecs <= 2) {
    launch_regs<DT, 2, kSample>(logits, p, k, min_p, out, B, V, ld, use_candidates, sa, stream);
  } else if (vecs <= 4) {
    launch_regs<DT, 4, kSample>(logits, p, k, min_p, out, B, V, ld, use_candidates, sa, stream);
  } else if (vecs <= 8) {
    launch_regs<DT, 8, kSample>(logits, p, k, min_p, out, B, V, ld, use_candidates, sa, stream);
  } else if (vecs <= 12) {
    launch_regs<DT, 12, kSample>(logits, p, k, min_p, out, B, V, ld, use_candidates, sa, stream);
  } else if (vecs <= 16) {
    launch_regs<DT, 16, kSample>(logits, p, k, min_p, out, B, V, ld, use_candidates, sa, stream);
  } else if (vecs <= 19) {
    launch_regs<DT, 19, kSample>(logits, p, k, min_p, out, B, V, ld, use_candidates, sa, stream);
  } else if constexpr (!kSample) {
    launch_regs<DT, kMaxVecs, kSample>(logits, p, k, min_p, out, B, V, ld, use_candidates, sa, stream);
  }
  return hipGetLastError();
}

// Any number of rows: launches of at most kMaxLaunchBlocks rows each, every
// pointer advanced to the launch's first row (the kernels index rows by
// block only).
template <class DT, bool kSample = false>
hipError_t launch_apply_t(const void* logits, const void* p, const int32_t* k, const void* min_p, void* out,
                          int64_t B, int64_t V, RowStrides ld, int policy, hipStream_t stream,
                          const SampleArgs& sa = SampleArgs{nullptr, 0, 0.0f, nullptr, nullptr, nullptr, nullptr, 0}) {
  using raw_t = typename DT::raw_t;
  for (int64_t r0 = 0; r0 < B; r0 += kMaxLaunchBlocks) {
    const int64_t nb = B - r0 < kMaxLaunchBlocks ? B - r0 : kMaxLaunchBlocks;
    SampleArgs s = sa;
    if (s.q != nullptr) s.q += r0 * s.ld_q;
    if (s.sel != nullptr) s.sel += r0;
    if (s.probs != nullptr) s.probs += r0 * s.cap;
    if (s.indices != nullptr) s.indices += r0 * s.cap;
    if (s.counts != nullptr) s.counts += r0;
    const hipError_t e = launch_apply_rows<DT, kSample>(
        static_cast<const raw_t*>(logits) + r0 * ld.x,
        p == nullptr ? nullptr : static_cast<const raw_t*>(p) + r0 * ld.pc,
        k == nullptr ? nullptr : k + r0 * ld.kc,
        min_p == nullptr ? nullptr : static_cast<const raw_t*>(min_p) + r0 * ld.mc,
        out == nullptr ? nullptr : static_cast<raw_t*>(out) + r0 * ld.o, nb, V, ld, policy, stream, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace tkp
