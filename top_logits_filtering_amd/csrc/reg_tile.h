// Row storage for the apply kernels: a slice of one row either held in
// registers (RegTile, NVEC 16-byte vectors per thread) or re-read from global
// memory on every traversal (GlobalTile). Both use one layout: element e of
// the slice lives in vector layer e / (1024 * P), thread (e % (1024 * P)) / P,
// lane e % P, with P elements per vector (4 for fp32, 8 for fp16/bf16).
// Consecutive threads touch consecutive 16-byte chunks, so each layer is one
// fully coalesced 16 KiB access per block, and a thread always writes the
// output addresses it read.
#pragma once

#include "device_common.h"

namespace tkp {

// Cache policy bits of the row loads and stores (gfx9 buffer instructions:
// 1 = sc0, 2 = nt, 16 = sc1). The row is read once: streaming (nt) loads.
// The output is not read again by the kernel: nontemporal stores as well.
constexpr int kLoadPolicy = 2;
constexpr int kStorePolicy = 2;

__device__ __forceinline__ uint32_t vword(const vec_t& q, int w) {
  return w == 0 ? q.x : (w == 1 ? q.y : (w == 2 ? q.z : q.w));
}
__device__ __forceinline__ void set_vword(vec_t& q, int w, uint32_t x) {
  if (w == 0) q.x = x;
  else if (w == 1) q.y = x;
  else if (w == 2) q.z = x;
  else q.w = x;
}
// Element j of a vector (j is a compile-time constant after unrolling).
template <class raw_t>
__device__ __forceinline__ raw_t lane_of(const vec_t& q, int j) {
  if constexpr (sizeof(raw_t) == 4) {
    return vword(q, j);
  } else {
    return static_cast<raw_t>(vword(q, j >> 1) >> ((j & 1) * 16));
  }
}
template <class raw_t>
__device__ __forceinline__ void set_lane(vec_t& q, int j, raw_t r) {
  if constexpr (sizeof(raw_t) == 4) {
    set_vword(q, j, r);
  } else {
    const int w = j >> 1, sh = (j & 1) * 16;
    set_vword(q, w, (vword(q, w) & ~(0xFFFFu << sh)) | (static_cast<uint32_t>(r) << sh));
  }
}
// Element j of a vector with a runtime j.
template <class raw_t>
__device__ __forceinline__ raw_t lane_of_dyn(const vec_t& q, int j) {
  if constexpr (sizeof(raw_t) == 4) {
    return q[j];
  } else {
    return static_cast<raw_t>(q[j >> 1] >> ((j & 1) * 16));
  }
}

__device__ __forceinline__ void store_vec(void* p, const vec_t& q) {
  vec_t* v = reinterpret_cast<vec_t*>(p);
  if constexpr ((kStorePolicy & 2) != 0) __builtin_nontemporal_store(q, v);
  else *v = q;
}

// threadIdx.x behind an empty asm, so per-element indices are recomputed in
// each traversal instead of being hoisted and kept alive in registers.
__device__ __forceinline__ int fresh_tid() {
  int t = static_cast<int>(threadIdx.x);
  asm volatile("" : "+v"(t));
  return t;
}

// Buffer resource word 3 for raw (untyped, stride-0) buffer access on gfx9.
constexpr int kRsrcWord3 = 0x00020000;

template <class raw_t>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const raw_t* p, int n) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<raw_t*>(p), static_cast<short>(0),
                                           n * static_cast<int>(sizeof(raw_t)), kRsrcWord3);
}

// A slice held in registers. All global accesses are raw buffer instructions
// on a descriptor bounded to the slice, so vectors past the slice end read
// as zero and their stores are dropped by the hardware: every lane issues
// exactly the same memory instructions, with no branches around them, and
// the compiler can count outstanding operations exactly (vector memory
// operations complete in order). Requires the slice start to be 16-byte
// aligned and its length a multiple of the vector width; launchers check this.
template <class DT, int NVEC>
struct RegTile {
  using raw_t = typename DT::raw_t;
  static constexpr bool kRegisters = true;
  static constexpr int kPV = DT::kPerVec;
  static constexpr int kSpan = kThreads * kPV;  // elements per vector layer
  static constexpr int kCapacity = NVEC * kSpan;
  static constexpr int kVecs = NVEC;
  static constexpr int kBytes = static_cast<int>(sizeof(raw_t)) * kPV;  // 16

  vec_t v[NVEC];
  int base;  // index of the slice's first element within the row
  int len;   // valid elements in the slice

  // Vector i as an opaque copy. Every traversal reads the tile through this,
  // so values derived from the tile in one traversal (keys, exponentials)
  // cannot be hoisted out of the selection loops and kept alive across
  // traversals, which would exhaust the register file.
  __device__ __forceinline__ vec_t fresh(int i) const {
    vec_t q = v[i];
    asm volatile("" : "+v"(q));
    return q;
  }

  __device__ __forceinline__ void load(const raw_t* __restrict__ row, int v0, int n) {
    base = v0;
    len = n;
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(row + v0, n);
    const int off = static_cast<int>(threadIdx.x) * kBytes;
#pragma unroll
    for (int i = 0; i < NVEC; ++i)
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, off + i * kSpan * static_cast<int>(sizeof(raw_t)), 0,
                                                   kLoadPolicy);
  }

  // f(i, q, e0) for every vector slot of this thread: q the data (zero past
  // the row end), e0 the slice index of its first element.
  template <class F>
  __device__ __forceinline__ void for_each_vec(F&& f) const {
    const int tid = fresh_tid();
#pragma unroll
    for (int i = 0; i < NVEC; ++i) f(i, fresh(i), i * kSpan + tid * kPV);
  }

  // f(i, e0) for every vector slot of this thread, without touching its data.
  template <class F>
  __device__ __forceinline__ void for_each_slot(F&& f) const {
    const int tid = fresh_tid();
#pragma unroll
    for (int i = 0; i < NVEC; ++i) f(i, i * kSpan + tid * kPV);
  }
  __device__ __forceinline__ vec_t vec_at(int i, int) const { return fresh(i); }

  // row[idx] = c for the elements of vector slot i of this thread.
  __device__ __forceinline__ void store_const_slot(raw_t* __restrict__ row, int i, raw_t c) const {
    vec_t cv = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < kPV; ++j) set_lane<raw_t>(cv, j, c);
    __builtin_amdgcn_raw_buffer_store_b128(cv, row_rsrc(row + base, len),
                                           fresh_tid() * kBytes + i * kSpan * static_cast<int>(sizeof(raw_t)), 0,
                                           kStorePolicy);
  }

  // row[idx] = c for every valid element of this thread, without its data.
  __device__ __forceinline__ void store_const(raw_t* __restrict__ row, raw_t c) const {
#pragma unroll
    for (int i = 0; i < NVEC; ++i) store_const_slot(row, i, c);
  }

  // The same for vector slots [I0, I1) only.
  template <int I0, int I1>
  __device__ __forceinline__ void store_const_range(raw_t* __restrict__ row, raw_t c) const {
#pragma unroll
    for (int i = I0; i < (I1 < NVEC ? I1 : NVEC); ++i) store_const_slot(row, i, c);
  }

  // f(raw, idx) for every valid element held by this thread; idx is the
  // element's index within the row.
  template <class F>
  __device__ __forceinline__ void for_each(F&& f) const {
    const int tid = fresh_tid();
#pragma unroll
    for (int i = 0; i < NVEC; ++i) {
      const int e0 = i * kSpan + tid * kPV;
      const vec_t q = fresh(i);
      if ((i + 1) * kSpan <= len) {  // whole layer valid: uniform over the block
#pragma unroll
        for (int j = 0; j < kPV; ++j) f(lane_of<raw_t>(q, j), base + e0 + j);
      } else {
#pragma unroll
        for (int j = 0; j < kPV; ++j)
          if (e0 + j < len) f(lane_of<raw_t>(q, j), base + e0 + j);
      }
    }
  }

  // f(i, x) for every vector slot of this thread, x[] holding the values as
  // fp32 with invalid slots (past the row end) set to -inf.
  template <int kB = 0, class F>  // (kB: the streamed tile's batch size; registers need none)
  __device__ __forceinline__ void for_each_vec_values(F&& f) const {
    const int tid = fresh_tid();
#pragma unroll
    for (int i = 0; i < NVEC; ++i) {
      const int e0 = i * kSpan + tid * kPV;
      float x[kPV];
      const vec_t q = fresh(i);
      if ((i + 1) * kSpan <= len) {
#pragma unroll
        for (int j = 0; j < kPV; ++j) x[j] = DT::value(lane_of<raw_t>(q, j));
      } else {
        const bool valid = e0 < len;  // whole vectors: the length is a multiple of the width
#pragma unroll
        for (int j = 0; j < kPV; ++j) x[j] = valid ? DT::value(lane_of<raw_t>(q, j)) : -INFINITY;
      }
      f(i, x);
    }
  }

  // Whole output vectors: g(q, e0) returns the vector stored for slot data q
  // whose first element is slice index e0.
  template <class G>
  __device__ __forceinline__ void store_vectors(raw_t* __restrict__ row, G&& g) const {
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(row + base, len);
    const int tid = fresh_tid();
#pragma unroll
    for (int i = 0; i < NVEC; ++i) {
      const int e0 = i * kSpan + tid * kPV;
      const vec_t o = g(fresh(i), e0);
      __builtin_amdgcn_raw_buffer_store_b128(o, rs, e0 * static_cast<int>(sizeof(raw_t)), 0, kStorePolicy);
    }
  }

  // row[idx] = g(raw, idx) for every valid element held by this thread.
  template <class G>
  __device__ __forceinline__ void store(raw_t* __restrict__ row, G&& g) const {
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(row + base, len);
    const int tid = fresh_tid();
#pragma unroll
    for (int i = 0; i < NVEC; ++i) {
      const int e0 = i * kSpan + tid * kPV;
      const vec_t q = fresh(i);
      vec_t o = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int j = 0; j < kPV; ++j) set_lane<raw_t>(o, j, g(lane_of<raw_t>(q, j), base + e0 + j));
      __builtin_amdgcn_raw_buffer_store_b128(o, rs, e0 * static_cast<int>(sizeof(raw_t)), 0, kStorePolicy);
    }
  }
};

// The same interface for rows too long to keep in registers: every traversal
// reads the row again from global memory, so later traversals mostly hit L2
// or the Infinity Cache. kStrided: element j of the row sits cs elements after
// element j - 1 (and of the output row ocs after), for views with a non-unit
// element stride; every access is then one element at a time.
template <class DT, bool kStrided = false>
struct GlobalTile {
  using raw_t = typename DT::raw_t;
  static constexpr bool kRegisters = false;
  static constexpr int kPV = DT::kPerVec;
  static constexpr int kSpan = kThreads * kPV;
  static constexpr int kVecs = 1;  // no per-vector state is kept for a streamed row

  const raw_t* src;
  int base;
  int len;
  bool aligned;
  bool vec_ok;  // 16-byte aligned and a whole number of vectors: bounded buffer loads
  int64_t cs = 1;   // element stride of the row (kStrided only)
  int64_t ocs = 1;  // element stride of the output row (kStrided only)

  __device__ __forceinline__ void load(const raw_t* __restrict__ row, int v0, int n) {
    src = row + v0;
    base = v0;
    len = n;
    aligned = !kStrided && (reinterpret_cast<uintptr_t>(src) & 15u) == 0;
    vec_ok = aligned && (n % kPV) == 0;
  }
  // kStrided: the row's element stride and the output row's
  __device__ __forceinline__ void load_strided(const raw_t* __restrict__ row, int n, int64_t stride,
                                               int64_t out_stride) {
    src = row;
    base = 0;
    len = n;
    aligned = false;
    vec_ok = false;
    cs = stride;
    ocs = out_stride;
  }
  __device__ __forceinline__ raw_t elem(int e) const {
    if constexpr (kStrided) return src[static_cast<int64_t>(e) * cs];
    else return src[e];
  }
  // the output element of row index idx, as an offset from the output row's start
  __device__ __forceinline__ int64_t out_at(int idx) const {
    if constexpr (kStrided) return static_cast<int64_t>(idx) * ocs;
    else return idx;
  }

  // Vector layers handled per batch by the first traversal: their loads are
  // issued together, so each thread keeps several requests in flight.
  static constexpr int kBatch = 8;

  // elements e0 .. e0+kPV-1 (zero past the end)
  __device__ __forceinline__ vec_t read(int e0) const {
    if (aligned && e0 + kPV <= len) return *reinterpret_cast<const vec_t*>(src + e0);
    vec_t q = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < kPV; ++j) set_lane<raw_t>(q, j, (e0 + j < len) ? elem(e0 + j) : static_cast<raw_t>(0));
    return q;
  }

  template <class F>
  __device__ __forceinline__ void for_each_vec(F&& f) const {
    int i = 0;
    for (int e0 = static_cast<int>(threadIdx.x) * kPV; e0 < len; e0 += kSpan, ++i) f(i, read(e0), e0);
  }

  template <class F>
  __device__ __forceinline__ void for_each_slot(F&& f) const {
    int i = 0;
    for (int e0 = static_cast<int>(threadIdx.x) * kPV; e0 < len; e0 += kSpan, ++i) f(i, e0);
  }
  __device__ __forceinline__ vec_t vec_at(int, int e0) const { return read(e0); }

  __device__ __forceinline__ void store_const(raw_t* __restrict__ row, raw_t c) const {
    if constexpr (kStrided) {
      for (int e = static_cast<int>(threadIdx.x); e < len; e += kThreads) row[out_at(base + e)] = c;
      return;
    }
    raw_t* dst = row + base;
    const bool dst_aligned = (reinterpret_cast<uintptr_t>(dst) & 15u) == 0;
    vec_t cv = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < kPV; ++j) set_lane<raw_t>(cv, j, c);
    for (int e0 = static_cast<int>(threadIdx.x) * kPV; e0 < len; e0 += kSpan) {
      if (dst_aligned && e0 + kPV <= len) {
        store_vec(dst + e0, cv);
      } else {
#pragma unroll
        for (int j = 0; j < kPV; ++j)
          if (e0 + j < len) dst[e0 + j] = c;
      }
    }
  }

  template <class F>
  __device__ __forceinline__ void for_each(F&& f) const {
#pragma unroll 2
    for (int e0 = static_cast<int>(threadIdx.x) * kPV; e0 < len; e0 += kSpan) {
      const vec_t q = read(e0);
#pragma unroll
      for (int j = 0; j < kPV; ++j)
        if (e0 + j < len) f(lane_of<raw_t>(q, j), base + e0 + j);
    }
  }

  // Vector e0 .. e0+kPV-1 of a candidate (e0 < len, a multiple of kPV).
  __device__ __forceinline__ vec_t gather(int e0) const {
    if (vec_ok)
      return __builtin_amdgcn_raw_buffer_load_b128(row_rsrc(src, len), e0 * static_cast<int>(sizeof(raw_t)), 0,
                                                   kLoadPolicy);
    return read(e0);
  }

  // kB: vector layers per batch (two batches in flight)
  template <int kB = kBatch, class F>
  __device__ __forceinline__ void for_each_vec_values(F&& f) const {
    if (vec_ok) {
      // two batches in flight: the next batch is requested before the
      // current one is consumed. Loads past the row end read zero and are
      // never consumed.
      const __amdgpu_buffer_rsrc_t rs = row_rsrc(src, len);
      const int tid = static_cast<int>(threadIdx.x);
      const int layers = (len + kSpan - 1) / kSpan;
      vec_t qa[kB], qb[kB];
      auto request = [&](vec_t(&q)[kB], int l0) {
#pragma unroll
        for (int u = 0; u < kB; ++u)
          q[u] = __builtin_amdgcn_raw_buffer_load_b128(
              rs, ((l0 + u) * kSpan + tid * kPV) * static_cast<int>(sizeof(raw_t)), 0, kLoadPolicy);
      };
      auto consume = [&](const vec_t(&q)[kB], int l0) {
#pragma unroll
        for (int u = 0; u < kB; ++u) {
          const int e0 = (l0 + u) * kSpan + tid * kPV;
          if (l0 + u < layers) {  // uniform: the layer exists
            float x[kPV];
#pragma unroll
            for (int j = 0; j < kPV; ++j) x[j] = (e0 + j < len) ? DT::value(lane_of<raw_t>(q[u], j)) : -INFINITY;
            f(l0 + u, x);
          }
        }
      };
      request(qa, 0);
      for (int l0 = 0; l0 < layers; l0 += 2 * kB) {
        request(qb, l0 + kB);
        consume(qa, l0);
        request(qa, l0 + 2 * kB);
        consume(qb, l0 + kB);
      }
      return;
    }
    int i = 0;
#pragma unroll 2
    for (int e0 = static_cast<int>(threadIdx.x) * kPV; e0 < len; e0 += kSpan, ++i) {
      const vec_t q = read(e0);
      float x[kPV];
#pragma unroll
      for (int j = 0; j < kPV; ++j) x[j] = (e0 + j < len) ? DT::value(lane_of<raw_t>(q, j)) : -INFINITY;
      f(i, x);
    }
  }

  template <class G>
  __device__ __forceinline__ void store(raw_t* __restrict__ row, G&& g) const {
    if constexpr (kStrided) {
      for (int e = static_cast<int>(threadIdx.x); e < len; e += kThreads) row[out_at(base + e)] = g(elem(e), base + e);
      return;
    }
    raw_t* dst = row + base;
    const bool dst_aligned = (reinterpret_cast<uintptr_t>(dst) & 15u) == 0;
#pragma unroll 2
    for (int e0 = static_cast<int>(threadIdx.x) * kPV; e0 < len; e0 += kSpan) {
      const vec_t q = read(e0);
      if (dst_aligned && e0 + kPV <= len) {
        vec_t o = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < kPV; ++j) set_lane<raw_t>(o, j, g(lane_of<raw_t>(q, j), base + e0 + j));
        store_vec(dst + e0, o);
      } else {
#pragma unroll
        for (int j = 0; j < kPV; ++j)
          if (e0 + j < len) dst[e0 + j] = g(lane_of<raw_t>(q, j), base + e0 + j);
      }
    }
  }
};

}  // namespace tkp
