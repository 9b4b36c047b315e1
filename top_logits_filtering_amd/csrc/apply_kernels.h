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
//  1. while the row arrives, each thread tracks the two largest of its
//     vector maxima and, for top-p rows without top-k, an online
//     (running-max rescaled) sum of exp(x - max);
//  2. the 2048 per-thread maxima are actual row elements, so the k-th largest
//     of them is a lower bound L on the top-k threshold; for top-p-only rows,
//     L is the key at which the mass of those maxima, walked from the top,
//     reaches (1 - t) * Z, so every element >= L carries at least that mass
//     and the top-p boundary cannot lie below L;
//  3. the whole output row is written as -inf right away (it does not depend
//     on the data), so these stores drain while the block works on;
//  4. every element >= L is appended to a shared-memory candidate list with a
//     wave ballot;
//  5. the exact selection (row_select.h) runs on the candidates only;
//  6. after the -inf stores have completed, the survivors are written over
//     them from the candidate list.
// Whenever a bound cannot be formed (k > 2048, top-p mass not reached) or the
// candidates overflow the list, the block falls back to the multi-pass plan,
// which rewrites the whole row; the same thread writes the same addresses in
// the same order, so the earlier -inf stores are overwritten.
//
// Multi-pass plan: the selection of row_select.h over every element of the
// row, re-read from global memory on each traversal (one per radix digit),
// then one coalesced write. Only the candidate plan's three traversals run
// over the register tile, which keeps the unrolled code small.

#pragma once

#include "launch.h"
#include "reg_tile.h"
#include "row_select.h"

namespace tkp {

constexpr int kCandCap = 8192;
constexpr int kTop2 = 2 * kThreads;
constexpr int kMaxVecs = 20;

// (raw, index) items held in shared memory.
template <class DT>
struct LdsItems {
  using raw_t = typename DT::raw_t;
  const uint32_t* raw;
  const uint32_t* idx;  // may be null: every index reads as 0
  int n;
  template <class F>
  __device__ __forceinline__ void for_each(F&& f) const {
    for (int c = threadIdx.x; c < n; c += kThreads)
      f(static_cast<raw_t>(raw[c]), idx != nullptr ? static_cast<int>(idx[c]) : 0);
  }
};

__device__ __forceinline__ double block_sum_f64(double v, RowSmem& sm, double* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) red[w] = v;
  __syncthreads();
  double r = 0.0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) r += red[i];
  __syncthreads();
  (void)sm;
  return r;
}

struct ApplySmem {
  RowSmem row;
  double redd[kWaves];
  uint32_t top2[kTop2];
  uint32_t cand_raw[kCandCap];
  uint32_t cand_idx[kCandCap];
  int ncand;
};

// Multi-pass plan over any tile, then one write of the whole row.
template <class DT, class Tile>
__device__ __forceinline__ void filter_multipass(const Tile& tile, const RowParams& rp, RowSmem& sm,
                                 typename DT::raw_t* __restrict__ orow) {
  using raw_t = typename DT::raw_t;
  uint32_t K, I;
  solve_row<DT>(tile, rp, sm, K, I);
  tile.store(orow, [K, I](raw_t r, int idx) {
    const uint32_t key = DT::key(r);
    return (key > K || (key == K && static_cast<uint32_t>(idx) >= I)) ? r : DT::kNegInf;
  });
}

// `tile` holds the row (registers or global); `irow` is the same row in
// global memory, re-read by the multi-pass fallback.
template <class DT, class Tile>
__device__ __forceinline__ void filter_row(const Tile& tile, const typename DT::raw_t* __restrict__ irow, int V,
                                           const RowParams& rp, bool use_candidates, ApplySmem& S,
                                           typename DT::raw_t* __restrict__ orow) {
  using raw_t = typename DT::raw_t;
  constexpr int kPV = DT::kPerVec;
  RowSmem& sm = S.row;
  GlobalTile<DT> gt;
  gt.load(irow, 0, V);

  if (!rp.k_on && rp.pmode == kPNone) {  // nothing to filter
    tile.store(orow, [](raw_t r, int) { return r; });
    return;
  }
  if (!use_candidates) {
    filter_multipass<DT>(gt, rp, sm, orow);
    return;
  }

  // 1. per-thread statistics
  const bool ponly = rp.pmode == kPBoundary && !rp.k_on;
  constexpr float kLog2e = 1.4426950408889634f;
  float M1 = -INFINITY, M2 = -INFINITY;  // two largest vector maxima of this thread
  float run = -INFINITY, acc = 0.0f;     // acc = sum of exp(x - run), ponly rows
  tile.for_each_vec_values([&](const float (&x)[kPV]) {
    float vm = x[0];
#pragma unroll
    for (int j = 1; j < kPV; ++j) vm = fmaxf(vm, x[j]);
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

  // 2. row maximum, per-thread maxima to shared memory, Z for top-p-only rows
  const float m = block_max_f32(M1, sm);
  S.top2[2 * threadIdx.x] = DT::raw_of_value(M1);
  S.top2[2 * threadIdx.x + 1] = DT::raw_of_value(M2);
  uint64_t thr = 0;
  if (ponly) {
    const double zt =
        (run > -INFINITY) ? static_cast<double>(acc) * static_cast<double>(__builtin_amdgcn_exp2f((run - m) * kLog2e))
                          : 0.0;
    const double Z = block_sum_f64(zt, sm, S.redd);  // >= 1: the maximum contributes exp(0)
    const uint64_t Zfx = static_cast<uint64_t>(Z * 8796093022208.0);  // 2^43
    thr = topp_threshold(rp.t, Zfx);
  }
  __syncthreads();

  // 3. candidate bound L
  const LdsItems<DT> top2{S.top2, nullptr, kTop2};
  const bool top_only = rp.pmode == kPTopOnly || (ponly && thr == 0);
  uint32_t L = 0;
  bool fast = true;
  if (rp.k_on) {
    fast = rp.k <= static_cast<uint32_t>(kTop2);
    if (fast)
      L = radix_select_desc(
          top2, DT::kKeyBits, rp.k, [](auto raw, int) { return DT::key(raw); }, [](auto, int) { return true; },
          sm);
  } else if (top_only) {
    L = DT::key(DT::raw_of_value(m));
  } else {
    uint64_t mt = 0;
    top2.for_each([&](auto raw, int) { mt += mass_fx(DT::value(raw), m); });
    mt = block_sum_u64(mt, sm);
    fast = mt >= thr;
    if (fast) {
      uint32_t Kb, Ib;
      topp_boundary<DT>(top2, 0u, m, thr, sm, Kb, Ib, false);
      L = Kb;
    }
  }
  if (!fast) {
    filter_multipass<DT>(gt, rp, sm, orow);
    return;
  }

  // 4. the whole row as -inf; these stores drain while the block continues
  tile.store(orow, [](raw_t, int) { return DT::kNegInf; });

  // 5. candidates: every element >= L (compared as values: -0.0 == +0.0)
  if (threadIdx.x == 0) S.ncand = 0;
  __syncthreads();
  const float Lf = DT::value(DT::raw_of_key(L));
  const int lane = threadIdx.x & (kWave - 1);
  tile.for_each([&](raw_t raw, int idx) {
    const bool c = DT::value(raw) >= Lf;
    const uint64_t mask = __ballot(c);
    if (mask != 0) {
      const int leader = __ffsll(static_cast<unsigned long long>(mask)) - 1;
      int base = 0;
      if (lane == leader) base = atomicAdd(&S.ncand, __popcll(mask));
      base = __shfl(base, leader);
      if (c) {
        const int pos = base + __popcll(mask & ((1ull << lane) - 1ull));
        if (pos < kCandCap) {
          S.cand_raw[pos] = raw;
          S.cand_idx[pos] = static_cast<uint32_t>(idx);
        }
      }
    }
  });
  __syncthreads();
  const int n = S.ncand;
  if (n > kCandCap) {
    filter_multipass<DT>(gt, rp, sm, orow);
    return;
  }

  // 6. exact selection on the candidates
  const LdsItems<DT> cs{S.cand_raw, S.cand_idx, n};
  uint32_t K = 0, I = 0;
  if (top_only && !rp.k_on) {
    top_position<DT>(cs, sm, K, I);
  } else {
    uint32_t Kk = 0;
    if (rp.k_on)
      Kk = radix_select_desc(
          cs, DT::kKeyBits, rp.k, [](auto raw, int) { return DT::key(raw); }, [](auto, int) { return true; }, sm);
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
        topp_boundary<DT>(cs, Kk, m, thr2, sm, K, I);
    } else {
      uint64_t a = 0;
      cs.for_each([&](auto raw, int) { a += mass_fx(DT::value(raw), m); });
      const uint64_t A = block_sum_u64(a, sm);
      if (A < thr) {  // the boundary lies below the candidates
        filter_multipass<DT>(gt, rp, sm, orow);
        return;
      }
      topp_boundary<DT>(cs, 0u, m, thr, sm, K, I);
    }
  }

  // 7. survivors over the -inf row, once every -inf store has completed
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int c = threadIdx.x; c < n; c += kThreads) {
    const raw_t raw = static_cast<raw_t>(S.cand_raw[c]);
    const uint32_t idx = S.cand_idx[c];
    const uint32_t key = DT::key(raw);
    if (key > K || (key == K && idx >= I)) orow[idx] = raw;
  }
}

template <class DT, int NVEC>
__global__ __launch_bounds__(kThreads) void apply_regs_kernel(const typename DT::raw_t* __restrict__ logits,
                                                              const typename DT::raw_t* __restrict__ p,
                                                              const int32_t* __restrict__ k,
                                                              typename DT::raw_t* __restrict__ out, int V,
                                                              int use_candidates) {
  __shared__ ApplySmem S;
  const int b = blockIdx.x;
  const size_t off = static_cast<size_t>(b) * V;
  RegTile<DT, NVEC> tile;
  tile.load(logits + off, 0, V);
  const RowParams rp = decode_row_params<DT>(p, k, b, V);
  filter_row<DT>(tile, logits + off, V, rp, use_candidates != 0, S, out + off);
}

template <class DT>
__global__ __launch_bounds__(kThreads) void apply_stream_kernel(const typename DT::raw_t* __restrict__ logits,
                                                                const typename DT::raw_t* __restrict__ p,
                                                                const int32_t* __restrict__ k,
                                                                typename DT::raw_t* __restrict__ out, int V,
                                                                int use_candidates) {
  __shared__ ApplySmem S;
  const int b = blockIdx.x;
  const size_t off = static_cast<size_t>(b) * V;
  GlobalTile<DT> tile;
  tile.load(logits + off, 0, V);
  const RowParams rp = decode_row_params<DT>(p, k, b, V);
  filter_row<DT>(tile, logits + off, V, rp, use_candidates != 0, S, out + off);
}

template <class DT, int NVEC>
void launch_regs(const void* logits, const void* p, const int32_t* k, void* out, int64_t B, int64_t V,
                        int use_candidates, hipStream_t stream) {
  using raw_t = typename DT::raw_t;
  hipLaunchKernelGGL((apply_regs_kernel<DT, NVEC>), dim3(static_cast<unsigned>(B)), dim3(kThreads), 0, stream,
                     static_cast<const raw_t*>(logits), static_cast<const raw_t*>(p), k, static_cast<raw_t*>(out),
                     static_cast<int>(V), use_candidates);
}

template <class DT>
hipError_t launch_apply_t(const void* logits, const void* p, const int32_t* k, void* out, int64_t B,
                                 int64_t V, int policy, hipStream_t stream) {
  using raw_t = typename DT::raw_t;
  constexpr int span = kThreads * DT::kPerVec;
  const int64_t vecs = (V + span - 1) / span;
  const int use_candidates = policy == kPlanGeneral ? 0 : 1;
  if (policy != kPlanAuto || vecs > kMaxVecs) {
    hipLaunchKernelGGL(apply_stream_kernel<DT>, dim3(static_cast<unsigned>(B)), dim3(kThreads), 0, stream,
                       static_cast<const raw_t*>(logits), static_cast<const raw_t*>(p), k, static_cast<raw_t*>(out),
                       static_cast<int>(V), use_candidates);
  } else if (vecs <= 1) {
    launch_regs<DT, 1>(logits, p, k, out, B, V, use_candidates, stream);
  } else if (vecs <= 2) {
    launch_regs<DT, 2>(logits, p, k, out, B, V, use_candidates, stream);
  } else if (vecs <= 4) {
    launch_regs<DT, 4>(logits, p, k, out, B, V, use_candidates, stream);
  } else if (vecs <= 8) {
    launch_regs<DT, 8>(logits, p, k, out, B, V, use_candidates, stream);
  } else if (vecs <= 12) {
    launch_regs<DT, 12>(logits, p, k, out, B, V, use_candidates, stream);
  } else if (vecs <= 16) {
    launch_regs<DT, 16>(logits, p, k, out, B, V, use_candidates, stream);
  } else if (vecs <= 19) {
    launch_regs<DT, 19>(logits, p, k, out, B, V, use_candidates, stream);
  } else {
    launch_regs<DT, kMaxVecs>(logits, p, k, out, B, V, use_candidates, stream);
  }
  return hipGetLastError();
}

}  // namespace tkp
