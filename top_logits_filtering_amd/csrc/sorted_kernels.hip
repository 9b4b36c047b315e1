// The sorted-input operator ApplyTopKTopPWithSorted (ApplyTopKTopPWithSorted
// guide, §1 and the §3 parameter table): sorted_value ascending,
// sorted_indices the permutation, p / k / logits optional.
//
// With the sort given, no selection is needed. Per row, in sorted positions:
//   * top-k: the threshold is sorted_value[V - k]; the first position holding
//     its key, `start`, is found by scanning down from V - k (equal values are
//     contiguous);
//   * top-p: Z sums the mass of positions [start, V); scanning down from the
//     top in 1024-position chunks with a block-wide prefix sum of the mass
//     gives F, the lowest position whose mass strictly above is below
//     (1 - t) * Z (a wave-level Kogge-Stone scan per chunk, in the spirit of
//     the guide's §6.3 CumsumKoggleStone / FindFirstIndex);
//   * min-p (aclnnTopKTopPSampleV2, "minP sampling"): its survivors are the
//     positions whose value passes exp(x - max) >= min_p, a suffix too, so F
//     moves up to the lowest of them when that is higher;
//   * survivors are the sorted positions >= F.
// With logits: out[v] = logits[v] when key(logits[v]) > key(s_F), -inf when
// below, and for equal keys the survivors are exactly the positions >= F of
// that run of equal values: the run's positions a..F-1 are collected into a
// shared-memory bitmap (the guide's ScatterBoundary idea) and masked, so the
// single coalesced pass over logits is the only full-row traffic.
// Without logits: the row is written as -inf, then the survivors are
// scattered over it, out[sorted_indices[j]] = sorted_value[j] for j >= F.
//
// Each row is split into slices handled by separate blocks; every block
// repeats the (cheap) boundary search, so no block waits on another and no
// global scratch is needed. The logits slice is loaded into registers before
// the boundary search so its latency overlaps that search. Without k the
// search scans the whole sorted row (Z needs every mass); that scan is bound
// by the vector ALUs (one exp2 per distinct value), so fewer blocks share a
// row then, each taking several slices.

#include <algorithm>
#include <type_traits>

#include "launch.h"
#include "reg_tile.h"

namespace tkp {

__device__ __forceinline__ int block_max_i32(int v, RowSmem& sm) {
  return static_cast<int>(block_max_u32(static_cast<uint32_t>(v + 1), sm)) - 1;
}

// Exclusive prefix sum over threadIdx.x; also returns the block total.
__device__ __forceinline__ uint64_t block_exscan_u64(uint64_t v, RowSmem& sm, uint64_t& total) {
  const int l = threadIdx.x & (kWave - 1);
  const int w = threadIdx.x / kWave;
  const uint64_t incl = wave_incl_scan_u64(v);
  if (l == kWave - 1) sm.redu[w] = incl;
  lds_barrier();
  const uint64_t x = l < kWaves ? sm.redu[l] : 0ull;
  const uint64_t wbase = wave_sum_u64(l < w ? x : 0ull);
  const uint64_t tot = wave_sum_u64(x);
  lds_barrier();
  total = tot;
  return wbase + incl - v;
}

// The sorted values of one row, read from global memory.
template <class DT>
struct SortedSrcGlobal {
  using raw_t = typename DT::raw_t;
  const raw_t* __restrict__ g;
  __device__ __forceinline__ raw_t at(int j) const { return g[j]; }
};

// Smallest j <= hi such that key(sv[j..hi]) >= K, given key(sv[hi]) >= K and
// an ascending row.
template <class DT, class Src>
__device__ __forceinline__ int first_at_or_above(const Src& sv, int hi, uint32_t K, RowSmem& sm) {
  int top = hi;
  for (;;) {
    const int j = top - 1 - static_cast<int>(threadIdx.x);
    const int cand = (j >= 0 && DT::key(sv.at(j)) < K) ? j : -1;
    const int best = block_max_i32(cand, sm);
    if (best >= 0) return best + 1;
    top -= kThreads;
    if (top <= 0) return 0;
  }
}

// Largest u64 and largest int over the block in one exchange round.
__device__ __forceinline__ void block_max_u64_i32(uint64_t a, int b, RowSmem& sm, uint64_t& amax, int& bmax) {
  a = wave_reduce_u64(a, 0ull, [](uint64_t x, uint64_t y) { return x > y ? x : y; });
  uint32_t bb = wave_max_u32(static_cast<uint32_t>(b + 1));
  const int l = threadIdx.x & (kWave - 1);
  if (l == 0) {
    sm.redu[threadIdx.x / kWave] = a;
    sm.redw[threadIdx.x / kWave] = bb;
  }
  lds_barrier();
  amax = wave_reduce_u64(l < kWaves ? sm.redu[l] : 0ull, 0ull, [](uint64_t x, uint64_t y) { return x > y ? x : y; });
  bmax = static_cast<int>(wave_max_u32(l < kWaves ? sm.redw[l] : 0u)) - 1;
  lds_barrier();
}

// Lowest sorted position F >= start whose mass strictly above is below
// (1 - t) * Z, with Z the mass of positions [start, V), read from global
// memory in two levels:
//   1. each thread sums the mass of one contiguous segment of groups, thread 0
//      taking the top segment (a group is one 16-byte vector when the row
//      allows vector loads, else one position);
//   2. an exclusive scan of the segment sums in thread order gives the mass
//      above each segment and Z; F lies in the lowest segment whose mass above
//      is below the threshold (every position under it has at least the
//      threshold above);
//   3. a block scan over that segment's positions (at most 1024 for
//      V <= 2^20) finds F.
// The masses are integers, so the result does not depend on how they are
// grouped. Returns V - 1 when the threshold is zero (t >= 1).
template <class DT, int kBatch>
__device__ __forceinline__ int topp_boundary_global(const typename DT::raw_t* __restrict__ sv, int start, int V,
                                                    float m, float t, RowSmem& sm) {
  using raw_t = typename DT::raw_t;
  constexpr int kPV = DT::kPerVec;
  const int tid = static_cast<int>(threadIdx.x);
  const bool vec = (V % kPV) == 0 && (reinterpret_cast<uintptr_t>(sv) & 15u) == 0;
  const int G = vec ? kPV : 1;              // positions per group
  const int gtop = (V - 1) / G;             // group of the top position
  const int glo = start / G;                // group of `start`
  const int L = (gtop - glo + kThreads) / kThreads;  // groups per segment
  const int g0 = gtop - tid * L;            // this thread: groups g0 down to g0 - L + 1, not below glo
  uint64_t s = 0;
  // the mass of a run of equal values is computed once per run (sorted rows
  // of 16-bit values are mostly long runs); no raw value equals ~0u here
  uint32_t prev = 0xFFFFFFFFu;
  uint64_t pe = 0;
  auto add = [&](raw_t r) {
    if (static_cast<uint32_t>(r) != prev) {
      pe = mass_fx(DT::value(r), m);
      prev = static_cast<uint32_t>(r);
    }
    s += pe;
  };
  if (vec) {
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(sv, V);
    for (int u0 = 0; u0 < L; u0 += kBatch) {
      vec_t q[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int g = g0 - u0 - u;
        q[u] = (u0 + u < L && g >= glo)
                   ? __builtin_amdgcn_raw_buffer_load_b128(rs, g * 16, 0, 0)
                   : vec_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int g = g0 - u0 - u;
        if (u0 + u < L && g >= glo) {
#pragma unroll
          for (int j = 0; j < kPV; ++j)
            if (g * kPV + j >= start) add(lane_of<raw_t>(q[u], j));
        }
      }
    }
  } else {
#pragma unroll 8
    for (int u = 0; u < L; ++u) {
      const int j = g0 - u;  // one position per group
      if (j >= glo) add(sv[j]);
    }
  }
  uint64_t Z;
  const uint64_t above = block_exscan_u64(s, sm, Z);
  const uint64_t thr = topp_threshold(t, Z);
  if (thr == 0) return V - 1;
  // the mass above a segment grows with the thread index: the largest mass
  // below the threshold is the one of the segment holding F
  const bool hit = g0 >= glo && above < thr;
  uint64_t base;
  int ts;
  block_max_u64_i32(hit ? above : 0ull, hit ? tid : -1, sm, base, ts);
  const int ptop = min(V - 1, (gtop - ts * L) * G + G - 1);
  const int pbot = max(start, (gtop - ts * L - L + 1) * G);
  const int j = ptop - tid;
  const bool valid = j >= pbot;
  const uint64_t e = valid ? mass_fx(DT::value(sv[j]), m) : 0ull;
  uint64_t total;
  const uint64_t excl = block_exscan_u64(e, sm, total);
  return ptop - block_max_i32(valid && base + excl < thr ? tid : -1, sm);
}

// Lowest sorted position j >= lo that survives min-p, given that the top
// position V-1 does (the decision is non-decreasing along the row). Level one
// tests 1024 positions spaced `stride` apart from the top; level two tests
// every position between the lowest passing sample and the sample below it.
template <class DT, class Src>
__device__ __forceinline__ int first_min_p(const Src& sv, int lo, int V, float minp, RowSmem& sm) {
  const float m = DT::value(sv.at(V - 1));
  const int stride = (V - lo + kThreads - 1) / kThreads;  // <= 1024 for V <= 2^20
  const int j = V - 1 - static_cast<int>(threadIdx.x) * stride;
  const bool pass = j >= lo && min_p_keeps(DT::value(sv.at(j)), m, minp);
  const int T = static_cast<int>(block_sum_u32(pass ? 1u : 0u, sm));  // samples 0..T-1 pass
  const int hi = V - 1 - (T - 1) * stride;  // lowest passing sample
  const int lo2 = max(lo, hi - stride + 1);
  if (lo2 >= hi) return hi;
  const int j2 = hi - 1 - static_cast<int>(threadIdx.x);
  const bool pass2 = j2 >= lo2 && min_p_keeps(DT::value(sv.at(j2)), m, minp);
  return hi - static_cast<int>(block_sum_u32(pass2 ? 1u : 0u, sm));
}

struct SortedBoundary {
  uint32_t KF;  // key of the lowest survivor
  int F;        // lowest surviving sorted position
  int a;        // first sorted position holding key KF (positions a..F-1 are masked)
};

template <class DT, int kScanBatch, class Src>
__device__ __forceinline__ SortedBoundary sorted_boundary(const Src& sv, const RowParams& rp, int V,
                                                          RowSmem& sm) {
  int start = 0;
  uint32_t Kk = 0;
  if (rp.k_on) {
    const int hi = V - static_cast<int>(rp.k);
    Kk = DT::key(sv.at(hi));
    start = first_at_or_above<DT>(sv, hi, Kk, sm);
  }
  int F = start;
  if (rp.pmode == kPTopOnly) {
    F = V - 1;
  } else if (rp.pmode == kPBoundary) {
    F = topp_boundary_global<DT, kScanBatch>(sv.g, start, V, DT::value(sv.at(V - 1)), rp.t, sm);
  }
  // min-p keeps a suffix of the sorted positions too: the tighter one wins
  if (rp.mp_on) F = first_min_p<DT>(sv, F, V, rp.minp, sm);
  SortedBoundary bd;
  bd.F = F;
  bd.KF = DT::key(sv.at(F));
  bd.a = (rp.k_on && bd.KF == Kk) ? start : first_at_or_above<DT>(sv, F, bd.KF, sm);
  return bd;
}

// Top sorted positions copied to shared memory before the slice loads; the
// copy serves rows whose k plus a margin for a run of values equal to the
// k-th largest fits in it.
constexpr int kSortedPrefetch = 6144;
constexpr int kSortedTieMargin = 1024;

// The same boundary from the copy of the top R sorted values in shared
// memory (position V - R + c at index c), for a top-k row whose run of values
// equal to the k-th largest starts inside the copy. Runs are found by each
// wave on its own (no barrier); the top-p walk gives every thread 8
// consecutive positions from the top, so one exclusive scan of their masses
// and one reduction find F.
template <class DT>
__device__ __forceinline__ int copy_run_start(const typename DT::raw_t* top, int c0, uint32_t K) {
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  for (int base = c0;; base -= kWave) {
    const int c = base - 1 - lane;
    const bool below = c < 0 || DT::key(top[c]) < K;
    const uint64_t m = __ballot(below);
    if (m != 0) return base - (__ffsll(static_cast<unsigned long long>(m)) - 1);
  }
}

template <class DT>
__device__ __forceinline__ SortedBoundary sorted_boundary_copy(const typename DT::raw_t* top, int R, int V,
                                                               const RowParams& rp, RowSmem& sm) {
  constexpr int G = kSortedPrefetch / kThreads;  // positions per thread in the top-p walk (the whole copy)
  const int ck = R - static_cast<int>(rp.k);
  const uint32_t Kk = DT::key(top[ck]);
  const int cs = copy_run_start<DT>(top, ck, Kk);
  int F = cs;
  if (rp.pmode == kPTopOnly) {
    F = R - 1;
  } else if (rp.pmode == kPBoundary) {
    // Only positions at or above cs hold mass: threads wholly below it (whole
    // waves, for all but the largest k) skip the exponentials, and only the
    // thread holding the boundary walks its positions one by one. Every
    // block of a row repeats this search, and the blocks resident on a
    // compute unit share its vector ALUs.
    const float m = DT::value(top[R - 1]);
    const int hi = R - G * static_cast<int>(threadIdx.x);  // this thread: positions hi-1 down to hi-G
    const bool live = hi > cs;                              // it holds a position at or above cs
    auto mass_at = [&](int c) { return mass_fx(DT::value(top[c]), m); };
    uint64_t tsum = 0, e_lo = 0;  // e_lo: mass of its lowest position at or above cs
    if (live) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int c = hi - 1 - g;
        if (c >= cs) {
          e_lo = mass_at(c);
          tsum += e_lo;
        }
      }
    }
    uint64_t Z;
    const uint64_t above = block_exscan_u64(tsum, sm, Z);  // threads run from the top down
    const uint64_t thr = topp_threshold(rp.t, Z);
    if (thr == 0) {
      F = R - 1;
    } else {
      int low = -1;  // this thread's lowest position whose mass strictly above is below thr
      if (live && above < thr) {
        if (above + (tsum - e_lo) < thr) {  // even its lowest position qualifies
          low = max(hi - G, cs);
        } else {  // the boundary lies among its positions
          uint64_t acc = above;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const int c = hi - 1 - g;
            if (c >= cs) {
              if (acc < thr) low = c;
              acc += mass_at(c);
            }
          }
        }
      }
      F = R - 1 - block_max_i32(low >= 0 ? R - 1 - low : -1, sm);
    }
  }
  if (rp.mp_on) {  // min-p survivors are a suffix of the copy: count them among the positions >= F
    const float m = DT::value(top[R - 1]);
    uint32_t c = 0;
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const int ci = u * kThreads + static_cast<int>(threadIdx.x);
      if (ci >= F && ci < R && min_p_keeps(DT::value(top[ci]), m, rp.minp)) ++c;
    }
    F = max(F, R - static_cast<int>(block_sum_u32(c, sm)));
  }
  SortedBoundary bd;
  bd.KF = DT::key(top[F]);
  bd.F = V - R + F;
  bd.a = V - R + (bd.KF == Kk ? cs : copy_run_start<DT>(top, F, bd.KF));
  return bd;
}

constexpr int kPre = kSortedPrefetch / kThreads;

// Requests the top R = min(V, 6144) sorted values of a row as bounded buffer
// loads of whole elements: no branch per load, so all of them are in flight
// together (positions past R read as zero and are never used).
template <class DT>
__device__ __forceinline__ void prefetch_top(const typename DT::raw_t* __restrict__ sv, int V, int R,
                                             typename DT::raw_t (&pre)[kPre]) {
  using raw_t = typename DT::raw_t;
  const __amdgpu_buffer_rsrc_t rs = row_rsrc(sv + (V - R), R);
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const int off = (u * kThreads + static_cast<int>(threadIdx.x)) * static_cast<int>(sizeof(raw_t));
    if constexpr (sizeof(raw_t) == 2)
      pre[u] = static_cast<raw_t>(__builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0));
    else
      pre[u] = static_cast<raw_t>(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
  }
}

// The search runs from the copy when the run of values equal to the k-th
// largest starts inside it (or the copy is the whole row).
template <class DT>
__device__ __forceinline__ bool boundary_from_copy(const typename DT::raw_t* top, int R, int V, const RowParams& rp) {
  return rp.k_on && (R == V || (static_cast<int>(rp.k) + kSortedTieMargin <= R &&
                                DT::key(top[0]) < DT::key(top[R - static_cast<int>(rp.k)])));
}

constexpr int kSortedVecs = 8;  // logits slice held in registers: 8 vectors per thread
constexpr int kMaxSliceWords = (kThreads * kSortedVecs * 8) / 32;

// Rows without k whose top-p boundary lies anywhere in the sorted row: Z needs
// the mass of every position, and every slice's block needs Z. A pre-pass
// (sorted_segment_mass_kernel) sums the mass of each segment of the sorted
// row once, and writes the row's table of segment masses into each slice's
// own region of the output row: the block of slice s reads the copy in its
// region and only then overwrites that region, so blocks never read what
// another block writes, and no memory beyond the caller's buffers is used. A
// slice too short to hold the table (the last one of some rows) searches the
// sorted row itself, as before. A segment is what one wave of the pre-pass
// reads: 8 vectors per lane, 4096 fp16/bf16 or 2048 fp32 positions.
template <class DT>
constexpr int seg_len() {
  return kWave * kSortedVecs * DT::kPerVec;
}

template <class DT>
__device__ __forceinline__ int segment_count(int V) {
  return (V + seg_len<DT>() - 1) / seg_len<DT>();  // <= 512 for V <= 2^20
}

// The table copy of slice s2 of a row, or NULL when the slice cannot hold it.
template <class DT>
__device__ __forceinline__ uint64_t* slice_table(typename DT::raw_t* orow, int s2, int V) {
  constexpr int kCap = RegTile<DT, kSortedVecs>::kCapacity;
  const int len = min(kCap, V - s2 * kCap);
  const bool fits = static_cast<int64_t>(len) * static_cast<int64_t>(sizeof(typename DT::raw_t)) >=
                    static_cast<int64_t>(segment_count<DT>(V)) * 8;
  return fits ? reinterpret_cast<uint64_t*>(orow + static_cast<size_t>(s2) * kCap) : nullptr;
}

// The summed mass of one 16-byte vector of sorted values (positions e0.. of a
// row of V, m the row maximum). A sorted vector is a run of its first value
// followed by a run of its last one unless it holds three or more distinct
// values (only in the thin tails of a row): then two masses times their
// counts give the same integer sum as the elements one by one.
template <class DT>
__device__ __forceinline__ uint64_t sorted_vector_mass(const vec_t& q, int e0, int V, float m) {
  using raw_t = typename DT::raw_t;
  constexpr int kPV = DT::kPerVec;
  const raw_t r0 = lane_of<raw_t>(q, 0), rl = lane_of<raw_t>(q, kPV - 1);
  uint32_t c0 = 0, cl = 0;
#pragma unroll
  for (int j = 0; j < kPV; ++j) {
    const raw_t r = lane_of<raw_t>(q, j);
    c0 += r == r0 ? 1u : 0u;
    cl += r == rl ? 1u : 0u;
  }
  if (e0 + kPV <= V && c0 + cl >= static_cast<uint32_t>(kPV)) {
    const uint64_t m0 = mass_fx(DT::value(r0), m);
    if (r0 == rl) return m0 * kPV;
    return m0 * c0 + mass_fx(DT::value(rl), m) * cl;
  }
  uint64_t sum = 0;
#pragma unroll
  for (int j = 0; j < kPV; ++j)
    if (e0 + j < V) sum += mass_fx(DT::value(lane_of<raw_t>(q, j)), m);
  return sum;
}

// Wave g of the grid sums the mass (mass_fx against the row maximum, the top
// sorted value) of one segment: segment g % nseg of row g / nseg. Its load u
// reads 64 consecutive vectors (1 KB), one wave sum gives the segment's mass,
// and lane 0 writes it into every table copy of the row. Waves share nothing,
// so blocks are small (4 waves) and need no barrier. Rows without a top-p
// boundary are skipped: the filter kernel reads no table for them.
constexpr int kSegWavesPerBlock = 4;

template <class DT>
__global__ __launch_bounds__(kSegWavesPerBlock * kWave) void sorted_segment_mass_kernel(
    const typename DT::raw_t* __restrict__ sorted_value, const typename DT::raw_t* __restrict__ p,
    const typename DT::raw_t* __restrict__ min_p, typename DT::raw_t* __restrict__ out, int64_t B, int V, int S,
    RowStrides ld) {
  using raw_t = typename DT::raw_t;
  constexpr int kPV = DT::kPerVec;
  constexpr int kSegLen = seg_len<DT>();
  const int nseg = segment_count<DT>(V);
  // the same in every lane: readfirstlane lets the compiler keep the row's
  // buffer descriptor in scalar registers
  const int64_t wg = static_cast<int64_t>(blockIdx.x) * kSegWavesPerBlock +
                     __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / kWave);
  if (wg >= B * nseg) return;  // uniform per wave
  const int b = static_cast<int>(wg / nseg);
  const int g = static_cast<int>(wg - static_cast<int64_t>(b) * nseg);
  const RowParams rp = decode_row_params<DT>(p, nullptr, min_p, b, V);
  if (rp.pmode != kPBoundary) return;
  const raw_t* __restrict__ sv = sorted_value + static_cast<size_t>(b) * static_cast<size_t>(ld.sv);
  raw_t* __restrict__ orow = out + static_cast<size_t>(b) * static_cast<size_t>(ld.o);
  const int lane = static_cast<int>(threadIdx.x) & (kWave - 1);
  const int e_seg = g * kSegLen;
  const __amdgpu_buffer_rsrc_t rs = row_rsrc(sv, V);
  // the row maximum is requested first: loads complete in order, so the
  // arithmetic on the first vectors need not wait for the last ones
  const raw_t top = sv[V - 1];
  __builtin_amdgcn_sched_barrier(0);
  vec_t q[kSortedVecs];
#pragma unroll
  for (int u = 0; u < kSortedVecs; ++u)
    q[u] = __builtin_amdgcn_raw_buffer_load_b128(
        rs, (e_seg + (u * kWave + lane) * kPV) * static_cast<int>(sizeof(raw_t)), 0, 0);
  const float m = DT::value(top);
  uint64_t sum = 0;
#pragma unroll
  for (int u = 0; u < kSortedVecs; ++u) sum += sorted_vector_mass<DT>(q[u], e_seg + (u * kWave + lane) * kPV, V, m);
  sum = wave_sum_u64(sum);
  if (lane < S) {  // lane s2 writes the copy of slice s2
    uint64_t* tab = slice_table<DT>(orow, lane, V);
    if (tab != nullptr) tab[g] = sum;
  }
}

// The top-p boundary of a row without k from its segment table (start 0):
// an exclusive scan of the segment masses from the top gives Z and the mass
// above each segment; F lies in the lowest segment whose mass above is below
// the threshold, and one block scan over that segment's positions (G
// consecutive positions per thread, from the top) finds it. The same integer
// masses as topp_boundary_global, so the same F.
template <class DT>
__device__ __forceinline__ int topp_boundary_table(const typename DT::raw_t* __restrict__ sv,
                                                   const uint64_t* __restrict__ tab, int V, float m, float t,
                                                   RowSmem& sm) {
  constexpr int kSegLen = seg_len<DT>();
  constexpr int G = kSegLen / kThreads;  // 4 or 2
  const int tid = static_cast<int>(threadIdx.x);
  const int nseg = segment_count<DT>(V);
  const int g = nseg - 1 - tid;  // thread tid takes the tid-th segment from the top
  const uint64_t ms = g >= 0 ? tab[g] : 0ull;
  uint64_t Z;
  const uint64_t above = block_exscan_u64(ms, sm, Z);
  const uint64_t thr = topp_threshold(t, Z);
  if (thr == 0) return V - 1;
  const bool hit = g >= 0 && above < thr;
  uint64_t base;
  int ts;
  block_max_u64_i32(hit ? above : 0ull, hit ? tid : -1, sm, base, ts);
  const int seg = nseg - 1 - ts;
  const int pbot = seg * kSegLen;
  const int ptop = min(V - 1, pbot + kSegLen - 1);
  const int hi = ptop - G * tid;  // this thread: positions hi down to hi - G + 1
  uint64_t e[G];
  uint64_t tsum = 0;
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int j = hi - i;
    e[i] = j >= pbot ? mass_fx(DT::value(sv[j]), m) : 0ull;
    tsum += e[i];
  }
  uint64_t total;
  uint64_t acc = base + block_exscan_u64(tsum, sm, total);  // mass strictly above position hi
  int low = -1;  // this thread's lowest position whose mass strictly above is below thr
#pragma unroll
  for (int i = 0; i < G; ++i) {
    const int j = hi - i;
    if (j >= pbot && acc < thr) low = j;
    acc += e[i];
  }
  return (V - 1) - block_max_i32(low >= 0 ? (V - 1) - low : -1, sm);
}

// kTable (with kRegs and kNoK): one block per slice, and rows with a top-p
// boundary take it from the segment table the pre-pass wrote.
template <class DT, bool kRegs, bool kNoK, bool kTable = false>
__global__ __launch_bounds__(kThreads, 8) void sorted_logits_kernel(
    const typename DT::raw_t* __restrict__ sorted_value, const int32_t* __restrict__ sorted_indices,
    const typename DT::raw_t* __restrict__ p, const int32_t* __restrict__ k,
    const typename DT::raw_t* __restrict__ min_p, const typename DT::raw_t* __restrict__ logits,
    typename DT::raw_t* __restrict__ out, int V, int S, RowStrides ld, int blocks_per_row) {
  using raw_t = typename DT::raw_t;
  using Tile = std::conditional_t<kRegs, RegTile<DT, kSortedVecs>, GlobalTile<DT>>;
  constexpr int kCap = RegTile<DT, kSortedVecs>::kCapacity;
  __shared__ RowSmem sm;
  __shared__ uint32_t ties[kMaxSliceWords];
  __shared__ __align__(16) raw_t top[kSortedPrefetch];

  // Without k (kNoK) no row can use the copy of the top values, and every
  // block of a row would scan the whole sorted row for Z: then Sb blocks
  // share the row's S slices (Sb = blocks_per_row, chosen so the batch still
  // fills the device), each taking its own run of slices one after another.
  const int Sb = kNoK ? blocks_per_row : S;
  const int b = static_cast<int>(blockIdx.x) / Sb;
  const int s = static_cast<int>(blockIdx.x) - b * Sb;
  const int s_lo = kNoK ? (s * S) / Sb : s;
  const int s_hi = kNoK ? ((s + 1) * S) / Sb : s + 1;
  int v0 = s_lo * kCap;
  int len = min(kCap, V - v0);
  const raw_t* __restrict__ sv = sorted_value + static_cast<size_t>(b) * static_cast<size_t>(ld.sv);

  // p[b] and k[b], the top sorted values the boundary search reads, then the
  // logits slice: vector loads complete in order, so the search waits only
  // for what it reads. The top values are requested before k is known.
  const RowParamsRaw<DT> rpr = fetch_row_params<DT>(p, k, min_p, b);
  const int R = min(V, kSortedPrefetch);
  raw_t pre[kPre];
  if constexpr (!kNoK) prefetch_top<DT>(sv, V, R, pre);
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the slice's
  Tile tile;
  if constexpr (!kNoK || kTable) tile.load(logits + static_cast<size_t>(b) * static_cast<size_t>(ld.x), v0, len);
  const RowParams rp = decode_row_params<DT>(rpr, V);
  if constexpr (!kNoK) {
#pragma unroll
    for (int u = 0; u < kPre; ++u) top[u * kThreads + threadIdx.x] = pre[u];  // entries past R: zero, unused
  }
  lds_barrier();

  raw_t* __restrict__ orow = out + static_cast<size_t>(b) * static_cast<size_t>(ld.o);
  const raw_t* __restrict__ xrow = logits + static_cast<size_t>(b) * static_cast<size_t>(ld.x);
  if (!row_filters(rp)) {
    if constexpr (kNoK && !kTable) {
      for (int ss = s_lo; ss < s_hi; ++ss) {
        v0 = ss * kCap;
        len = min(kCap, V - v0);
        tile.load(xrow, v0, len);
        tile.store(orow, [](raw_t r, int) { return r; });
      }
    } else {
      tile.store(orow, [](raw_t r, int) { return r; });
    }
    return;
  }
  SortedBoundary bd;
  if constexpr (kTable) {
    const uint64_t* tab = slice_table<DT>(out + static_cast<size_t>(b) * static_cast<size_t>(ld.o), s, V);
    if (rp.pmode == kPBoundary && tab != nullptr) {
      int F = topp_boundary_table<DT>(sv, tab, V, DT::value(sv[V - 1]), rp.t, sm);
      if (rp.mp_on) F = first_min_p<DT>(SortedSrcGlobal<DT>{sv}, F, V, rp.minp, sm);
      bd.F = F;
      bd.KF = DT::key(sv[F]);
      bd.a = first_at_or_above<DT>(SortedSrcGlobal<DT>{sv}, F, bd.KF, sm);
    } else {
      // (fp16 keeps one scan load fewer in flight beside the slice tile, as below)
      bd = sorted_boundary<DT, std::is_same_v<DT, F16T> ? 3 : 4>(SortedSrcGlobal<DT>{sv}, rp, V, sm);
    }
  } else if constexpr (kNoK) {
    bd = sorted_boundary<DT, 8>(SortedSrcGlobal<DT>{sv}, rp, V, sm);
  } else if (boundary_from_copy<DT>(top, R, V, rp)) {
    bd = sorted_boundary_copy<DT>(top, R, V, rp, sm);
  } else {
    // the slice tile is live beside the scan: fp16, whose conversions take
    // more registers, keeps one load fewer in flight so nothing spills
    constexpr int kScan = std::is_same_v<DT, F16T> && kRegs ? 3 : 4;
    bd = sorted_boundary<DT, kScan>(SortedSrcGlobal<DT>{sv}, rp, V, sm);
  }

  const int32_t* __restrict__ si = sorted_indices + static_cast<size_t>(b) * static_cast<size_t>(ld.si);
  for (int ss = s_lo; ss < s_hi; ++ss) {
  if constexpr (kNoK && !kTable) {
    v0 = ss * kCap;
    len = min(kCap, V - v0);
    tile.load(xrow, v0, len);
    if (ss > s_lo) lds_barrier();  // the previous slice's bitmap reads are done
  }
  const int words = (len + 31) / 32;
  for (int i = threadIdx.x; i < words; i += kThreads) ties[i] = 0;
  lds_barrier();
  for (int j = bd.a + static_cast<int>(threadIdx.x); j < bd.F; j += kThreads) {
    const int v = si[j] - v0;
    if (v >= 0 && v < len) atomicOr(&ties[v >> 5], 1u << (v & 31));
  }
  lds_barrier();

  const uint32_t KF = bd.KF;
  if (bd.a == bd.F) {  // no member of the lowest survivor's run is masked
    tile.store(orow, [&](raw_t r, int) { return DT::key(r) >= KF ? r : DT::kNegInf; });
  } else if constexpr (kRegs) {
    // the masked flags of a vector's elements sit in one bitmap word
    tile.store_vectors(orow, [&](const vec_t& q, int e0) {
      const uint32_t w = ties[e0 >> 5] >> (e0 & 31);
      vec_t o = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < DT::kPerVec; ++j) {
        const raw_t r = lane_of<raw_t>(q, j);
        const uint32_t key = DT::key(r);
        const bool keep = key > KF || (key == KF && ((w >> j) & 1u) == 0);
        set_lane<raw_t>(o, j, keep ? r : DT::kNegInf);
      }
      return o;
    });
  } else {
    tile.store(orow, [&](raw_t r, int idx) {
      const uint32_t key = DT::key(r);
      bool keep = key > KF;
      if (key == KF) {
        const int v = idx - v0;
        keep = ((ties[v >> 5] >> (v & 31)) & 1u) == 0;
      }
      return keep ? r : DT::kNegInf;
    });
  }
  }
}

constexpr int kScatterSlice = 65536;

// Without logits: out[sorted_indices[j]] = j >= F ? sorted_value[j] : -inf.
// Block s of a row owns output positions [s * 65536, (s + 1) * 65536). It
// requests the row's top sorted values first (as the logits kernel does),
// writes its slice as -inf with coalesced stores, finds F while they drain,
// waits for them, and writes the survivors (sorted positions F..V-1) whose
// index falls in its slice. Only the survivors' values and indices
// are read, instead of the whole permutation. A row with nothing to filter
// is a plain scatter, each block taking a slice of the sorted positions.
template <class DT>
__global__ __launch_bounds__(kThreads) void sorted_scatter_kernel(
    const typename DT::raw_t* __restrict__ sorted_value, const int32_t* __restrict__ sorted_indices,
    const typename DT::raw_t* __restrict__ p, const int32_t* __restrict__ k,
    const typename DT::raw_t* __restrict__ min_p, typename DT::raw_t* __restrict__ out, int V, int S,
    RowStrides ld) {
  using raw_t = typename DT::raw_t;
  constexpr int kPV = DT::kPerVec;
  __shared__ RowSmem sm;
  __shared__ __align__(16) raw_t top[kSortedPrefetch];
  const int b = blockIdx.x / S;
  const int s = blockIdx.x - b * S;
  const auto* __restrict__ sv = sorted_value + static_cast<size_t>(b) * static_cast<size_t>(ld.sv);
  const int32_t* __restrict__ si = sorted_indices + static_cast<size_t>(b) * static_cast<size_t>(ld.si);
  raw_t* __restrict__ orow = out + static_cast<size_t>(b) * static_cast<size_t>(ld.o);
  const int v0 = s * kScatterSlice;
  const int v1 = min(V, v0 + kScatterSlice);

  const RowParamsRaw<DT> rpr = fetch_row_params<DT>(p, k, min_p, b);
  const int R = min(V, kSortedPrefetch);
  raw_t pre[kPre];
  prefetch_top<DT>(sv, V, R, pre);
  __builtin_amdgcn_sched_barrier(0);  // keep these loads ahead of the stores below
  const RowParams rp = decode_row_params<DT>(rpr, V);
  if (!row_filters(rp)) {  // nothing to filter: a plain scatter of sorted positions [v0, v1)
    for (int j = v0 + static_cast<int>(threadIdx.x); j < v1; j += kThreads) {
      const int v = si[j];
      if (static_cast<unsigned>(v) < static_cast<unsigned>(V)) orow[v] = sv[j];
    }
    return;
  }
#pragma unroll
  for (int u = 0; u < kPre; ++u) top[u * kThreads + threadIdx.x] = pre[u];  // entries past R: zero, unused

  // The output slice as -inf, in two portions: a quarter before the boundary
  // search (it drains while the search runs on the shared-memory copy) and
  // the rest after the survivors' loads are issued (a wave stalls at its
  // stores once the memory pipeline is full, and loads issued after stores
  // complete after them).
  raw_t* dst = orow + v0;
  const int n = v1 - v0;
  const bool vec_out = (reinterpret_cast<uintptr_t>(dst) & 15u) == 0;
  const int nv = vec_out ? n / kPV : 0;  // whole 16-byte vectors
  vec_t cv = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < kPV; ++j) set_lane<raw_t>(cv, j, DT::kNegInf);
  const __amdgpu_buffer_rsrc_t rs = row_rsrc(dst, n);
  const int nv_a = nv / 4;
  for (int e = static_cast<int>(threadIdx.x); e < nv_a; e += kThreads)
    __builtin_amdgcn_raw_buffer_store_b128(cv, rs, e * 16, 0, kStorePolicy);
  for (int e = nv * kPV + static_cast<int>(threadIdx.x); e < n; e += kThreads) dst[e] = DT::kNegInf;
  lds_barrier();  // the copy is in place (this barrier does not wait for the stores)

  const int F = boundary_from_copy<DT>(top, R, V, rp) ? sorted_boundary_copy<DT>(top, R, V, rp, sm).F
                                                      : sorted_boundary<DT, 4>(SortedSrcGlobal<DT>{sv}, rp, V, sm).F;
  // The survivors, 8 per thread per round with every load of a round in
  // flight together (bounded buffer loads: positions past V read as zero).
  // The first round's loads are issued before the wait for the -inf stores,
  // so they arrive while those stores drain.
  constexpr int kRound = 8;
  const int ns = V - F;
  const __amdgpu_buffer_rsrc_t ri = row_rsrc(si + F, ns);
  const __amdgpu_buffer_rsrc_t rv = row_rsrc(sv + F, ns);
  int vv[kRound];
  raw_t xv[kRound];
  auto request = [&](int c0) {
#pragma unroll
    for (int u = 0; u < kRound; ++u) {
      const int c = c0 + u * kThreads + static_cast<int>(threadIdx.x);
      vv[u] = __builtin_amdgcn_raw_buffer_load_b32(ri, c * 4, 0, 0);
      if constexpr (sizeof(raw_t) == 2)
        xv[u] = static_cast<raw_t>(__builtin_amdgcn_raw_buffer_load_b16(rv, c * 2, 0, 0));
      else
        xv[u] = static_cast<raw_t>(__builtin_amdgcn_raw_buffer_load_b32(rv, c * 4, 0, 0));
    }
  };
  request(0);
  for (int e = nv_a + static_cast<int>(threadIdx.x); e < nv; e += kThreads)
    __builtin_amdgcn_raw_buffer_store_b128(cv, rs, e * 16, 0, kStorePolicy);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int c0 = 0; c0 < ns; c0 += kRound * kThreads) {
    if (c0 > 0) request(c0);
#pragma unroll
    for (int u = 0; u < kRound; ++u) {
      const int c = c0 + u * kThreads + static_cast<int>(threadIdx.x);
      if (c < ns && vv[u] >= v0 && vv[u] < v1) orow[vv[u]] = xv[u];
    }
  }
}

// Rows [0, B) in one launch (B times the blocks per row <= kMaxLaunchBlocks).
template <class DT>
static hipError_t launch_sorted_rows(const void* sorted_value, const int32_t* sorted_indices, const void* p,
                                     const int32_t* k, const void* min_p, const void* logits, void* out, int64_t B,
                                     int64_t V, RowStrides ld, hipStream_t stream) {
  using raw_t = typename DT::raw_t;
  if (logits != nullptr) {
    constexpr int cap = RegTile<DT, kSortedVecs>::kCapacity;
    const int S = static_cast<int>((V + cap - 1) / cap);
    constexpr int64_t es = static_cast<int64_t>(sizeof(raw_t));
    const bool vec_ok = (V % DT::kPerVec) == 0 && (reinterpret_cast<uintptr_t>(logits) & 15u) == 0 &&
                        (reinterpret_cast<uintptr_t>(out) & 15u) == 0 && (ld.x * es) % 16 == 0 &&
                        (ld.o * es) % 16 == 0;
    // without k: blocks per row so that the batch still fills the 256 CUs
    const int Sb = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(S, 256 / std::max<int64_t>(B, 1))));
    auto go = [&](auto kernel, int64_t grid) {
      hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream,
                         static_cast<const raw_t*>(sorted_value), sorted_indices, static_cast<const raw_t*>(p), k,
                         static_cast<const raw_t*>(min_p), static_cast<const raw_t*>(logits), static_cast<raw_t*>(out),
                         static_cast<int>(V), S, ld, Sb);
    };
    // without k no row can use the copy of the top values: no copy; with p,
    // the pre-pass sums the sorted rows' segment masses once (one block per
    // slice), otherwise the slices are read after each block's own search
    const bool sv_vec = (reinterpret_cast<uintptr_t>(sorted_value) & 15u) == 0 && (ld.sv * es) % 16 == 0;
    if (vec_ok && sv_vec && k == nullptr && p != nullptr) {
      // one wave per segment: seg_len() positions per segment, four waves per block
      const int64_t seg_waves = B * ((V + seg_len<DT>() - 1) / seg_len<DT>());
      hipLaunchKernelGGL(sorted_segment_mass_kernel<DT>,
                         dim3(static_cast<unsigned>((seg_waves + kSegWavesPerBlock - 1) / kSegWavesPerBlock)),
                         dim3(kSegWavesPerBlock * kWave), 0, stream, static_cast<const raw_t*>(sorted_value),
                         static_cast<const raw_t*>(p), static_cast<const raw_t*>(min_p), static_cast<raw_t*>(out), B,
                         static_cast<int>(V), S, ld);
      hipLaunchKernelGGL((sorted_logits_kernel<DT, true, true, true>), dim3(static_cast<unsigned>(B * S)),
                         dim3(kThreads), 0, stream, static_cast<const raw_t*>(sorted_value), sorted_indices,
                         static_cast<const raw_t*>(p), k, static_cast<const raw_t*>(min_p),
                         static_cast<const raw_t*>(logits), static_cast<raw_t*>(out), static_cast<int>(V), S, ld, S);
    } else if (vec_ok && k == nullptr)
      go(sorted_logits_kernel<DT, true, true>, B * Sb);
    else if (vec_ok)
      go(sorted_logits_kernel<DT, true, false>, B * S);
    else if (k == nullptr)
      go(sorted_logits_kernel<DT, false, true>, B * Sb);
    else
      go(sorted_logits_kernel<DT, false, false>, B * S);
  } else {
    const int S = static_cast<int>((V + kScatterSlice - 1) / kScatterSlice);
    hipLaunchKernelGGL(sorted_scatter_kernel<DT>, dim3(static_cast<unsigned>(B * S)), dim3(kThreads), 0, stream,
                       static_cast<const raw_t*>(sorted_value), sorted_indices, static_cast<const raw_t*>(p), k,
                       static_cast<const raw_t*>(min_p), static_cast<raw_t*>(out), static_cast<int>(V), S, ld);
  }
  return hipGetLastError();
}

// Blocks per row of the launches above (at most: rows without k may take fewer).
template <class DT>
static int64_t sorted_blocks_per_row(int64_t V, bool with_logits) {
  constexpr int64_t cap = RegTile<DT, kSortedVecs>::kCapacity;
  return with_logits ? (V + cap - 1) / cap : (V + kScatterSlice - 1) / kScatterSlice;
}

// Any number of rows: launches of at most kMaxLaunchBlocks blocks each, every
// pointer advanced to the launch's first row.
template <class DT>
static hipError_t launch_sorted_t(const void* sorted_value, const int32_t* sorted_indices, const void* p,
                                  const int32_t* k, const void* min_p, const void* logits, void* out, int64_t B,
                                  int64_t V, RowStrides ld, hipStream_t stream) {
  using raw_t = typename DT::raw_t;
  const int64_t rows = kMaxLaunchBlocks / sorted_blocks_per_row<DT>(V, logits != nullptr);
  for (int64_t r0 = 0; r0 < B; r0 += rows) {
    const int64_t nb = B - r0 < rows ? B - r0 : rows;
    const hipError_t e = launch_sorted_rows<DT>(
        static_cast<const raw_t*>(sorted_value) + r0 * ld.sv, sorted_indices + r0 * ld.si,
        p == nullptr ? nullptr : static_cast<const raw_t*>(p) + r0, k == nullptr ? nullptr : k + r0,
        min_p == nullptr ? nullptr : static_cast<const raw_t*>(min_p) + r0,
        logits == nullptr ? nullptr : static_cast<const raw_t*>(logits) + r0 * ld.x, static_cast<raw_t*>(out) + r0 * ld.o,
        nb, V, ld, stream);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_with_sorted(int dtype, const void* sorted_value, const int32_t* sorted_indices, const void* p,
                              const int32_t* k, const void* min_p, const void* logits, void* out, int64_t B,
                              int64_t V, RowStrides ld, hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_sorted_t<F32T>(sorted_value, sorted_indices, p, k, min_p, logits, out, B, V, ld, stream);
    case 1: return launch_sorted_t<F16T>(sorted_value, sorted_indices, p, k, min_p, logits, out, B, V, ld, stream);
    case 2: return launch_sorted_t<BF16T>(sorted_value, sorted_indices, p, k, min_p, logits, out, B, V, ld, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tkp
