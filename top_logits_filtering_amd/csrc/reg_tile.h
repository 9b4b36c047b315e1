// A slice of one row held in registers: NVEC 16-byte vectors per thread.
// Element e of the slice lives in vector layer e / (1024 * P), thread
// (e % (1024 * P)) / P, lane e % P, with P elements per vector (4 for fp32, 8
// for fp16/bf16). Consecutive threads therefore touch consecutive 16-byte
// chunks, and each layer is one fully coalesced 16 KiB access per block.
// All loops are unrolled at compile time so the array stays in VGPRs.
#pragma once

#include "device_common.h"

namespace tkp {

template <class DT, int NVEC>
struct RegTile {
  using raw_t = typename DT::raw_t;
  static constexpr int kPV = DT::kPerVec;
  static constexpr int kSpan = kThreads * kPV;  // elements per vector layer
  static constexpr int kCapacity = NVEC * kSpan;

  uint4 v[NVEC];
  int base;  // index of the slice's first element within the row
  int len;   // valid elements in the slice

  // Element access by (vector, lane). Both indices are compile-time constants
  // after unrolling, so these fold to register moves and shifts.
  static __device__ __forceinline__ uint32_t word(const uint4& q, int w) {
    return w == 0 ? q.x : (w == 1 ? q.y : (w == 2 ? q.z : q.w));
  }
  static __device__ __forceinline__ void set_word(uint4& q, int w, uint32_t x) {
    if (w == 0) q.x = x;
    else if (w == 1) q.y = x;
    else if (w == 2) q.z = x;
    else q.w = x;
  }
  static __device__ __forceinline__ raw_t lane_of(const uint4& q, int j) {
    if constexpr (sizeof(raw_t) == 4) {
      return word(q, j);
    } else {
      return static_cast<raw_t>(word(q, j >> 1) >> ((j & 1) * 16));
    }
  }
  static __device__ __forceinline__ void set_lane(uint4& q, int j, raw_t r) {
    if constexpr (sizeof(raw_t) == 4) {
      set_word(q, j, r);
    } else {
      const int w = j >> 1, sh = (j & 1) * 16;
      set_word(q, w, (word(q, w) & ~(0xFFFFu << sh)) | (static_cast<uint32_t>(r) << sh));
    }
  }
  __device__ __forceinline__ raw_t get(int i, int j) const { return lane_of(v[i], j); }
  __device__ __forceinline__ void set(int i, int j, raw_t r) { set_lane(v[i], j, r); }

  // Vector i as an opaque copy. Every traversal reads the tile through this,
  // so values derived from the tile in one traversal (keys, exponentials)
  // cannot be hoisted out of the selection loops and kept alive across
  // traversals, which would exhaust the register file.
  __device__ __forceinline__ uint4 fresh(int i) const {
    uint4 q = v[i];
    asm volatile("" : "+v"(q.x), "+v"(q.y), "+v"(q.z), "+v"(q.w));
    return q;
  }
  // threadIdx.x behind the same barrier, so per-element indices are
  // recomputed in each traversal instead of living in registers throughout.
  static __device__ __forceinline__ int fresh_tid() {
    int t = static_cast<int>(threadIdx.x);
    asm volatile("" : "+v"(t));
    return t;
  }

  __device__ __forceinline__ void load(const raw_t* __restrict__ row, int v0, int n) {
    base = v0;
    len = n;
    const raw_t* src = row + v0;
    const bool aligned = (reinterpret_cast<uintptr_t>(src) & 15u) == 0;
#pragma unroll
    for (int i = 0; i < NVEC; ++i) {
      const int e0 = i * kSpan + static_cast<int>(threadIdx.x) * kPV;
      if (aligned && e0 + kPV <= n) {
        v[i] = *reinterpret_cast<const uint4*>(src + e0);
      } else {
#pragma unroll
        for (int j = 0; j < kPV; ++j) set(i, j, (e0 + j < n) ? src[e0 + j] : static_cast<raw_t>(0));
      }
    }
  }

  // f(raw, idx) for every valid element held by this thread; idx is the
  // element's index within the row.
  template <class F>
  __device__ __forceinline__ void for_each(F&& f) const {
    const int tid = fresh_tid();
#pragma unroll
    for (int i = 0; i < NVEC; ++i) {
      const int e0 = i * kSpan + tid * kPV;
      const uint4 q = fresh(i);
      if ((i + 1) * kSpan <= len) {  // whole layer valid: uniform over the block
#pragma unroll
        for (int j = 0; j < kPV; ++j) f(lane_of(q, j), base + e0 + j);
      } else {
#pragma unroll
        for (int j = 0; j < kPV; ++j)
          if (e0 + j < len) f(lane_of(q, j), base + e0 + j);
      }
    }
  }

  // f(x) for every vector held by this thread, x[] holding the values as
  // fp32 with invalid slots (past the row end) set to -inf.
  template <class F>
  __device__ __forceinline__ void for_each_vec_values(F&& f) const {
    const int tid = fresh_tid();
#pragma unroll
    for (int i = 0; i < NVEC; ++i) {
      const int e0 = i * kSpan + tid * kPV;
      float x[kPV];
      const uint4 q = fresh(i);
      if ((i + 1) * kSpan <= len) {
#pragma unroll
        for (int j = 0; j < kPV; ++j) x[j] = DT::value(lane_of(q, j));
      } else {
#pragma unroll
        for (int j = 0; j < kPV; ++j) x[j] = (e0 + j < len) ? DT::value(lane_of(q, j)) : -INFINITY;
      }
      f(x);
    }
  }

  // row[idx] = g(raw, idx) for every valid element held by this thread.
  template <class G>
  __device__ __forceinline__ void store(raw_t* __restrict__ row, G&& g) const {
    raw_t* dst = row + base;
    const bool aligned = (reinterpret_cast<uintptr_t>(dst) & 15u) == 0;
    const int tid = fresh_tid();
#pragma unroll
    for (int i = 0; i < NVEC; ++i) {
      const int e0 = i * kSpan + tid * kPV;
      const uint4 q = fresh(i);
      if (aligned && e0 + kPV <= len) {
        uint4 o = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int j = 0; j < kPV; ++j) set_lane(o, j, g(lane_of(q, j), base + e0 + j));
        *reinterpret_cast<uint4*>(dst + e0) = o;
      } else {
#pragma unroll
        for (int j = 0; j < kPV; ++j)
          if (e0 + j < len) dst[e0 + j] = g(lane_of(q, j), base + e0 + j);
      }
    }
  }
};

}  // namespace tkp

namespace tkp {

// The same interface as RegTile for rows too long to keep in registers: every
// traversal reads the row again from global memory (16-byte loads, the same
// element-to-thread layout), so later traversals mostly hit L2 or the
// Infinity Cache.
template <class DT>
struct GlobalTile {
  using raw_t = typename DT::raw_t;
  static constexpr int kPV = DT::kPerVec;
  static constexpr int kSpan = kThreads * kPV;

  const raw_t* src;
  int base;
  int len;
  bool aligned;

  __device__ __forceinline__ void load(const raw_t* __restrict__ row, int v0, int n) {
    src = row + v0;
    base = v0;
    len = n;
    aligned = (reinterpret_cast<uintptr_t>(src) & 15u) == 0;
  }

  // raw elements e0 .. e0+kPV-1 (zero past the end)
  __device__ __forceinline__ void read(int e0, raw_t (&r)[kPV]) const {
    if (aligned && e0 + kPV <= len) {
      const uint4 q = *reinterpret_cast<const uint4*>(src + e0);
#pragma unroll
      for (int j = 0; j < kPV; ++j) r[j] = RegTile<DT, 1>::lane_of(q, j);
    } else {
#pragma unroll
      for (int j = 0; j < kPV; ++j) r[j] = (e0 + j < len) ? src[e0 + j] : static_cast<raw_t>(0);
    }
  }

  template <class F>
  __device__ __forceinline__ void for_each(F&& f) const {
#pragma unroll 2
    for (int e0 = static_cast<int>(threadIdx.x) * kPV; e0 < len; e0 += kSpan) {
      raw_t r[kPV];
      read(e0, r);
#pragma unroll
      for (int j = 0; j < kPV; ++j)
        if (e0 + j < len) f(r[j], base + e0 + j);
    }
  }

  template <class F>
  __device__ __forceinline__ void for_each_vec_values(F&& f) const {
#pragma unroll 2
    for (int e0 = static_cast<int>(threadIdx.x) * kPV; e0 < len; e0 += kSpan) {
      raw_t r[kPV];
      read(e0, r);
      float x[kPV];
#pragma unroll
      for (int j = 0; j < kPV; ++j) x[j] = (e0 + j < len) ? DT::value(r[j]) : -INFINITY;
      f(x);
    }
  }

  template <class G>
  __device__ __forceinline__ void store(raw_t* __restrict__ row, G&& g) const {
    raw_t* dst = row + base;
    const bool dst_aligned = (reinterpret_cast<uintptr_t>(dst) & 15u) == 0;
#pragma unroll 2
    for (int e0 = static_cast<int>(threadIdx.x) * kPV; e0 < len; e0 += kSpan) {
      raw_t r[kPV];
      read(e0, r);
      if (dst_aligned && e0 + kPV <= len) {
        uint4 o = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int j = 0; j < kPV; ++j) RegTile<DT, 1>::set_lane(o, j, g(r[j], base + e0 + j));
        *reinterpret_cast<uint4*>(dst + e0) = o;
      } else {
#pragma unroll
        for (int j = 0; j < kPV; ++j)
          if (e0 + j < len) dst[e0 + j] = g(r[j], base + e0 + j);
      }
    }
  }
};

}  // namespace tkp
