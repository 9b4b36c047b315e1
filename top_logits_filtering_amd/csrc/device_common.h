// Device-side building blocks of the top-k / top-p filter (gfx950, wave64).
//
// Notation. A row holds V values x[0..V). key(x) is a 32-bit unsigned image of
// x that is monotone in IEEE float order with -0.0 and +0.0 given the same key
// (the stable ascending sort of the filter treats them as equal). The filter's
// result for a row is always a suffix of the stable ascending order, which is
// fully described by a pair (K, I): keep x[v] iff key(x[v]) > K, or
// key(x[v]) == K and v >= I. Every kernel computes that pair without sorting.
//
// Probability mass is carried as 64-bit fixed point with 43 fraction bits:
// mass(x) = floor(exp(x - m) * 2^43) with m the row maximum, so mass <= 2^43
// and a row of up to 2^20 values sums below 2^63. Integer sums are exact and
// independent of summation order, which keeps the output deterministic from
// run to run whatever order the hardware adds in.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tkp {

// Workgroup barrier for shared-memory communication only: it orders this
// wave's shared-memory accesses around the barrier but does not wait for its
// outstanding global loads and stores (a plain __syncthreads() waits for all
// of them, which would tie every step to the -inf stores still draining).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// 16 bytes: the unit of row loads and stores and of shared-memory vector access.
using vec_t = uint32_t __attribute__((ext_vector_type(4)));


constexpr int kThreads = 1024;           // threads per row-block
constexpr int kWave = 64;                // gfx950 wavefront
constexpr int kWaves = kThreads / kWave; // 16
constexpr int kMassShift = 43;

// ---------------------------------------------------------------- dtypes ----

struct F32T {
  using raw_t = uint32_t;
  static constexpr int kKeyBits = 32;
  static constexpr raw_t kNegInf = 0xFF800000u;
  static constexpr int kPerVec = 4;  // elements per 16-byte vector
  __device__ static __forceinline__ float value(raw_t r) { return __uint_as_float(r); }
  __device__ static __forceinline__ uint32_t key(raw_t r) {
    uint32_t u = (r == 0x80000000u) ? 0u : r;  // -0.0 -> +0.0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  }
  // inverse of key() (zero comes back as +0.0)
  __device__ static __forceinline__ raw_t raw_of_key(uint32_t K) { return (K & 0x80000000u) ? (K & 0x7FFFFFFFu) : ~K; }
  // bits of a value known to be representable in this dtype
  __device__ static __forceinline__ raw_t raw_of_value(float f) { return __float_as_uint(f); }
  // 16-bit upper bound of a value (bf16 rounded toward +inf) and its value
  __device__ static __forceinline__ uint32_t ub16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0xFFFFu) != 0u && (u & 0x80000000u) == 0u) u += 0x10000u;
    return u >> 16;
  }
  __device__ static __forceinline__ float ub16_value(uint32_t h) { return __uint_as_float(h << 16); }
};

struct F16T {
  using raw_t = uint16_t;
  static constexpr int kKeyBits = 16;
  static constexpr raw_t kNegInf = 0xFC00u;
  static constexpr int kPerVec = 8;
  __device__ static __forceinline__ float value(raw_t r) {
    return static_cast<float>(__builtin_bit_cast(_Float16, r));
  }
  __device__ static __forceinline__ uint32_t key(raw_t r) {
    uint32_t u = (r == 0x8000u) ? 0u : r;
    return (u & 0x8000u) ? (~u & 0xFFFFu) : (u | 0x8000u);
  }
  __device__ static __forceinline__ raw_t raw_of_key(uint32_t K) {
    return static_cast<raw_t>((K & 0x8000u) ? (K & 0x7FFFu) : (~K & 0xFFFFu));
  }
  __device__ static __forceinline__ raw_t raw_of_value(float f) {
    return __builtin_bit_cast(raw_t, static_cast<_Float16>(f));
  }
  // values are fp16 already: the 16-bit form is exact
  __device__ static __forceinline__ uint32_t ub16(float f) { return raw_of_value(f); }
  __device__ static __forceinline__ float ub16_value(uint32_t h) { return value(static_cast<raw_t>(h)); }
};

struct BF16T {
  using raw_t = uint16_t;
  static constexpr int kKeyBits = 16;
  static constexpr raw_t kNegInf = 0xFF80u;
  static constexpr int kPerVec = 8;
  __device__ static __forceinline__ float value(raw_t r) { return __uint_as_float(static_cast<uint32_t>(r) << 16); }
  __device__ static __forceinline__ uint32_t key(raw_t r) {
    uint32_t u = (r == 0x8000u) ? 0u : r;
    return (u & 0x8000u) ? (~u & 0xFFFFu) : (u | 0x8000u);
  }
  __device__ static __forceinline__ raw_t raw_of_key(uint32_t K) {
    return static_cast<raw_t>((K & 0x8000u) ? (K & 0x7FFFu) : (~K & 0xFFFFu));
  }
  __device__ static __forceinline__ raw_t raw_of_value(float f) { return static_cast<raw_t>(__float_as_uint(f) >> 16); }
  __device__ static __forceinline__ uint32_t ub16(float f) { return raw_of_value(f); }
  __device__ static __forceinline__ float ub16_value(uint32_t h) { return value(static_cast<raw_t>(h)); }
};

// exp(x - m) as 43-bit fixed point, for x <= m. Uses the hardware exp2; the
// relative error of a term is about |x - m| * 1e-7, far below the 1e-5 band in
// which top-p decisions may differ from an exact evaluation.
__device__ __forceinline__ uint64_t mass_fx(float x, float m) {
  float e = __builtin_amdgcn_exp2f((x - m) * 1.4426950408889634f);
  e = fminf(e, 1.0f);
  float hi_f = e * 2048.0f;  // 2^11, exact
  uint32_t hi = static_cast<uint32_t>(hi_f);
  float frac = hi_f - static_cast<float>(hi);  // exact
  uint32_t lo = static_cast<uint32_t>(frac * 4294967296.0f);
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

// ------------------------------------------------------------- reductions ---
// Wave-wide reductions and scans with DPP lane moves (gfx9 encodings), which
// stay in the VALU instead of going through the LDS crossbar:
//   quad_perm [1,0,3,2] and [2,3,0,1] combine within quads, row_half_mirror and
//   row_mirror within 8 and 16 lanes, row_shr:n shifts within a 16-lane row,
//   row_bcast:15 / row_bcast:31 carry a row's last lane into the following
//   rows. Lanes a move does not write (row_mask) or whose source is outside the
//   row receive `old`, which is always the operation's identity here.

namespace dpp {
constexpr int kQuad1032 = 0xB1;
constexpr int kQuad2301 = 0x4E;
constexpr int kRowMirror = 0x140;
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;
constexpr int kRowShr1 = 0x111;
constexpr int kRowShr2 = 0x112;
constexpr int kRowShr4 = 0x114;
constexpr int kRowShr8 = 0x118;
}  // namespace dpp

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, uint32_t old) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(static_cast<int>(old), static_cast<int>(v), CTRL, ROW_MASK, 0xF, false));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v, uint64_t old) {
  const uint32_t lo = dpp_u32<CTRL, ROW_MASK>(static_cast<uint32_t>(v), static_cast<uint32_t>(old));
  const uint32_t hi = dpp_u32<CTRL, ROW_MASK>(static_cast<uint32_t>(v >> 32), static_cast<uint32_t>(old >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

__device__ __forceinline__ uint32_t lane63_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}
// Number of set bits of a wave-uniform lane mask below the calling lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0u));
}
__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int lane) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), lane));
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
  return (static_cast<uint64_t>(readlane_u32(static_cast<uint32_t>(v >> 32), lane)) << 32) |
         readlane_u32(static_cast<uint32_t>(v), lane);
}
__device__ __forceinline__ uint64_t lane63_u64(uint64_t v) {
  return (static_cast<uint64_t>(lane63_u32(static_cast<uint32_t>(v >> 32))) << 32) |
         lane63_u32(static_cast<uint32_t>(v));
}

// Reduction of v over the wave with a commutative, associative op and its
// identity; the result is uniform (every lane gets it).
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, uint32_t id, Op op) {
  v = op(v, dpp_u32<dpp::kQuad1032>(v, id));
  v = op(v, dpp_u32<dpp::kQuad2301>(v, id));
  v = op(v, dpp_u32<dpp::kRowHalfMirror>(v, id));
  v = op(v, dpp_u32<dpp::kRowMirror>(v, id));
  v = op(v, dpp_u32<dpp::kRowBcast15, 0xA>(v, id));
  v = op(v, dpp_u32<dpp::kRowBcast31, 0x8>(v, id));
  return lane63_u32(v);
}
template <class Op>
__device__ __forceinline__ uint64_t wave_reduce_u64(uint64_t v, uint64_t id, Op op) {
  v = op(v, dpp_u64<dpp::kQuad1032>(v, id));
  v = op(v, dpp_u64<dpp::kQuad2301>(v, id));
  v = op(v, dpp_u64<dpp::kRowHalfMirror>(v, id));
  v = op(v, dpp_u64<dpp::kRowMirror>(v, id));
  v = op(v, dpp_u64<dpp::kRowBcast15, 0xA>(v, id));
  v = op(v, dpp_u64<dpp::kRowBcast31, 0x8>(v, id));
  return lane63_u64(v);
}

// Inclusive prefix sums over the lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  v += dpp_u32<dpp::kRowShr1>(v, 0u);
  v += dpp_u32<dpp::kRowShr2>(v, 0u);
  v += dpp_u32<dpp::kRowShr4>(v, 0u);
  v += dpp_u32<dpp::kRowShr8>(v, 0u);
  v += dpp_u32<dpp::kRowBcast15, 0xA>(v, 0u);
  v += dpp_u32<dpp::kRowBcast31, 0xC>(v, 0u);
  return v;
}
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v) {
  v += dpp_u64<dpp::kRowShr1>(v, 0ull);
  v += dpp_u64<dpp::kRowShr2>(v, 0ull);
  v += dpp_u64<dpp::kRowShr4>(v, 0ull);
  v += dpp_u64<dpp::kRowShr8>(v, 0ull);
  v += dpp_u64<dpp::kRowBcast15, 0xA>(v, 0ull);
  v += dpp_u64<dpp::kRowBcast31, 0xC>(v, 0ull);
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
  const uint32_t r = wave_reduce_u32(__float_as_uint(v), __float_as_uint(-INFINITY), [](uint32_t a, uint32_t b) {
    return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b)));
  });
  return __uint_as_float(r);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce_u32(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  return wave_reduce_u32(v, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
  return wave_reduce_u64(v, 0ull, [](uint64_t a, uint64_t b) { return a + b; });
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return wave_reduce_u32(v, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  const uint64_t r = wave_reduce_u64(__builtin_bit_cast(uint64_t, v), 0ull, [](uint64_t a, uint64_t b) {
    return __builtin_bit_cast(uint64_t, __builtin_bit_cast(double, a) + __builtin_bit_cast(double, b));
  });
  return __builtin_bit_cast(double, r);
}

// Shared-memory workspace for block reductions and broadcasts.
struct RowSmem {
  float redf[kWaves];
  uint64_t redu[kWaves];
  uint32_t redw[kWaves];
};

// Block-wide reductions: one DPP reduction per wave, the 16 wave results
// through shared memory, and a second DPP reduction in which lane i holds
// wave i's result (lanes >= 16 hold the identity). Every thread gets the
// result. Two barriers, the second one so the slots can be reused.

__device__ __forceinline__ float block_max_f32(float v, RowSmem& sm) {
  v = wave_max_f32(v);
  const int l = threadIdx.x & (kWave - 1);
  if (l == 0) sm.redf[threadIdx.x / kWave] = v;
  lds_barrier();
  const float r = wave_max_f32(l < kWaves ? sm.redf[l] : -INFINITY);
  lds_barrier();
  return r;
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, RowSmem& sm) {
  v = wave_max_u32(v);
  const int l = threadIdx.x & (kWave - 1);
  if (l == 0) sm.redw[threadIdx.x / kWave] = v;
  lds_barrier();
  const uint32_t r = wave_max_u32(l < kWaves ? sm.redw[l] : 0u);
  lds_barrier();
  return r;
}

__device__ __forceinline__ uint32_t block_min_u32(uint32_t v, RowSmem& sm) {
  v = wave_min_u32(v);
  const int l = threadIdx.x & (kWave - 1);
  if (l == 0) sm.redw[threadIdx.x / kWave] = v;
  lds_barrier();
  const uint32_t r = wave_min_u32(l < kWaves ? sm.redw[l] : 0xFFFFFFFFu);
  lds_barrier();
  return r;
}

// max of a float and min of a u32 in one exchange round
__device__ __forceinline__ void block_max_f32_min_u32(float a, uint32_t b, RowSmem& sm, float& amax,
                                                      uint32_t& bmin) {
  a = wave_max_f32(a);
  b = wave_min_u32(b);
  const int l = threadIdx.x & (kWave - 1);
  if (l == 0) {
    sm.redf[threadIdx.x / kWave] = a;
    sm.redw[threadIdx.x / kWave] = b;
  }
  lds_barrier();
  amax = wave_max_f32(l < kWaves ? sm.redf[l] : -INFINITY);
  bmin = wave_min_u32(l < kWaves ? sm.redw[l] : 0xFFFFFFFFu);
  lds_barrier();
}

__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, RowSmem& sm) {
  v = wave_sum_u64(v);
  const int l = threadIdx.x & (kWave - 1);
  if (l == 0) sm.redu[threadIdx.x / kWave] = v;
  lds_barrier();
  const uint64_t r = wave_sum_u64(l < kWaves ? sm.redu[l] : 0ull);
  lds_barrier();
  return r;
}

__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, RowSmem& sm) {
  v = wave_sum_u32(v);
  const int l = threadIdx.x & (kWave - 1);
  if (l == 0) sm.redw[threadIdx.x / kWave] = v;
  lds_barrier();
  const uint32_t r = wave_sum_u32(l < kWaves ? sm.redw[l] : 0u);
  lds_barrier();
  return r;
}

// ------------------------------------------------------------- row modes ---

enum PMode : int { kPNone = 0, kPTopOnly = 1, kPBoundary = 2 };

struct RowParams {
  bool k_on;     // 1 <= k <= V-1
  uint32_t k;
  int pmode;     // kPNone: no top-p (p absent, or t <= 0); kPTopOnly: t >= 1, or min_p >= 1
  float t;       // 1 - p in fp32
  bool mp_on;    // 0 < min_p < 1: the min-p stage masks positions with exp(x - max) < min_p
  float minp;
};

// The per-row parameters are the same for every thread of the block. They are
// fetched first (fetch_row_params) and decoded later (decode_row_params), so a
// kernel can put its row loads in between: vector loads complete in order, and
// waiting for p[b] and k[b] must not mean waiting for the row. Decoded values
// live in scalar registers.
template <class DT>
struct RowParamsRaw {
  int32_t k;
  typename DT::raw_t p, mp;
  bool has_k, has_p, has_mp;
};

template <class DT>
__device__ __forceinline__ RowParamsRaw<DT> fetch_row_params(const typename DT::raw_t* p, const int32_t* k,
                                                             const typename DT::raw_t* min_p, int b) {
  RowParamsRaw<DT> r;
  r.has_k = k != nullptr;
  r.has_p = p != nullptr;
  r.has_mp = min_p != nullptr;
  r.k = r.has_k ? k[b] : 0;
  r.p = r.has_p ? p[b] : static_cast<typename DT::raw_t>(0);
  r.mp = r.has_mp ? min_p[b] : static_cast<typename DT::raw_t>(0);
  return r;
}

// The same for parameter vectors whose entries are pc, kc and mc elements apart.
template <class DT>
__device__ __forceinline__ RowParamsRaw<DT> fetch_row_params_strided(const typename DT::raw_t* p, const int32_t* k,
                                                                     const typename DT::raw_t* min_p, int64_t b,
                                                                     int64_t pc, int64_t kc, int64_t mc) {
  RowParamsRaw<DT> r;
  r.has_k = k != nullptr;
  r.has_p = p != nullptr;
  r.has_mp = min_p != nullptr;
  r.k = r.has_k ? k[b * kc] : 0;
  r.p = r.has_p ? p[b * pc] : static_cast<typename DT::raw_t>(0);
  r.mp = r.has_mp ? min_p[b * mc] : static_cast<typename DT::raw_t>(0);
  return r;
}

template <class DT>
__device__ __forceinline__ RowParams decode_row_params(const RowParamsRaw<DT>& r, int V) {
  RowParams rp;
  rp.k_on = false;
  rp.k = 0;
  if (r.has_k) {
    const int32_t kb = __builtin_amdgcn_readfirstlane(r.k);
    if (kb >= 1 && kb <= V - 1) {
      rp.k_on = true;
      rp.k = static_cast<uint32_t>(kb);
    }
  }
  rp.pmode = kPNone;
  rp.t = 0.0f;
  if (r.has_p) {
    const float pb = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(DT::value(r.p))));
    const float t = 1.0f - pb;
    rp.t = t;
    if (t >= 1.0f) rp.pmode = kPTopOnly;
    else if (t > 0.0f) rp.pmode = kPBoundary;
    // t <= 0 (p >= 1) or NaN: no position with positive mass is masked
  }
  // min-p (aclnnTopKTopPSampleV2, "minP sampling"): min_p >= 1 keeps one
  // token with the maximum value, the same single survivor as t >= 1; min_p
  // <= 0 (or NaN) skips the stage
  rp.mp_on = false;
  rp.minp = 0.0f;
  if (r.has_mp) {
    const float mp = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(DT::value(r.mp))));
    if (mp >= 1.0f) {
      rp.pmode = kPTopOnly;
    } else if (mp > 0.0f) {
      rp.mp_on = true;
      rp.minp = mp;
    }
  }
  return rp;
}

template <class DT>
__device__ __forceinline__ RowParams decode_row_params(const typename DT::raw_t* p, const int32_t* k,
                                                       const typename DT::raw_t* min_p, int b, int V) {
  return decode_row_params<DT>(fetch_row_params<DT>(p, k, min_p, b), V);
}

// Largest key whose value is <= f (f finite).
template <class DT>
__device__ __forceinline__ uint32_t key_floor(float f) {
  uint32_t K = DT::key(DT::raw_of_value(f));  // within one step of the answer
  if (K > 0u && DT::value(DT::raw_of_key(K)) > f) --K;
  return K;
}

// The row filters something (top-k, top-p or min-p is active).
__device__ __forceinline__ bool row_filters(const RowParams& rp) {
  return rp.k_on || rp.pmode != kPNone || rp.mp_on;
}

// Min-p decision of one value: exp(x - m) >= min_p, with the exponential
// taken as in mass_fx (hardware exp2 of (x - m) * log2 e). Non-decreasing in x.
__device__ __forceinline__ bool min_p_keeps(float x, float m, float minp) {
  return __builtin_amdgcn_exp2f((x - m) * 1.4426950408889634f) >= minp;
}

// A value below which nothing passes min_p_keeps: m + ln(min_p), widened by
// a margin far above the error of the exponential.
__device__ __forceinline__ float min_p_floor(float m, float minp) {
  const float l2 = log2f(minp);  // <= 0
  return m + (l2 * 1.0009765625f - 0.0009765625f) * 0.6931471805599453f;
}

// Fixed-point threshold: a position survives top-p iff the mass strictly above
// it (in the stable descending order) is below (1 - t) * Z; for an integer
// mass D that is D < ceil((1 - t) * Z). The result never exceeds Z.
__device__ __forceinline__ uint64_t topp_threshold(float t, uint64_t Z) {
  double thr_d = ceil((1.0 - static_cast<double>(t)) * static_cast<double>(Z));
  if (!(thr_d > 0.0)) return 0;
  if (thr_d >= static_cast<double>(Z)) return Z;
  uint64_t thr = static_cast<uint64_t>(thr_d);
  return thr < Z ? thr : Z;
}

}  // namespace tkp
