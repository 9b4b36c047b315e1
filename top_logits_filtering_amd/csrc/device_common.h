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

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t w = __shfl_xor(v, o);
    v = v > w ? v : w;
  }
  return v;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Shared-memory workspace of one row-block.
struct RowSmem {
  uint32_t hist[256];   // digit counts
  uint64_t mhist[256];  // digit mass (fixed point)
  float redf[kWaves];
  uint64_t redu[kWaves];
  uint32_t redw[kWaves];
  // result of a bin search, broadcast to the block
  int sel_bin;
  uint32_t sel_above;    // count strictly above the selected bin
  uint64_t sel_above64;  // mass strictly above the selected bin
  uint32_t sel_cnt;      // count in the selected bin
  uint64_t sel_mass;     // mass in the selected bin
  uint32_t bcast[4];
};

__device__ __forceinline__ float block_max_f32(float v, RowSmem& sm) {
  v = wave_max_f32(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) sm.redf[w] = v;
  __syncthreads();
  float r = sm.redf[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = fmaxf(r, sm.redf[i]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, RowSmem& sm) {
  v = wave_max_u32(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) sm.redw[w] = v;
  __syncthreads();
  uint32_t r = sm.redw[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) r = r > sm.redw[i] ? r : sm.redw[i];
  __syncthreads();
  return r;
}

__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, RowSmem& sm) {
  v = wave_sum_u64(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) sm.redu[w] = v;
  __syncthreads();
  uint64_t r = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) r += sm.redu[i];
  __syncthreads();
  return r;
}

__device__ __forceinline__ uint32_t block_sum_u32(uint32_t v, RowSmem& sm) {
  v = wave_sum_u32(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x & (kWave - 1)) == 0) sm.redw[w] = v;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) r += sm.redw[i];
  __syncthreads();
  return r;
}

// ------------------------------------------------------------ bin search ---
// Walks the 256 bins from the highest down and selects the first bin whose
// inclusive running total reaches `target` (target >= 1). Wave 0 does the walk
// with a wave-wide prefix sum (lane l owns bins 255-4l .. 252-4l); the result
// lands in sm.sel_* and is visible to the whole block after the call. If the
// target exceeds the grand total, bin 0 is selected.

__device__ __forceinline__ void select_bin_count(RowSmem& sm, uint32_t target) {
  if (threadIdx.x < kWave) {
    const int l = threadIdx.x;
    const int b0 = 255 - 4 * l;
    uint32_t c0 = sm.hist[b0], c1 = sm.hist[b0 - 1], c2 = sm.hist[b0 - 2], c3 = sm.hist[b0 - 3];
    uint32_t tot = c0 + c1 + c2 + c3;
    uint32_t incl = tot;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      uint32_t n = __shfl_up(incl, o);
      if (l >= o) incl += n;
    }
    uint32_t excl = incl - tot;
    bool hit = (excl < target && target <= incl) || (l == kWave - 1 && target > incl);
    if (hit) {
      uint32_t a = excl;
      int bin;
      uint32_t cnt;
      if (a + c0 >= target) { bin = b0; cnt = c0; }
      else { a += c0;
        if (a + c1 >= target) { bin = b0 - 1; cnt = c1; }
        else { a += c1;
          if (a + c2 >= target) { bin = b0 - 2; cnt = c2; }
          else { a += c2; bin = b0 - 3; cnt = c3; } } }
      sm.sel_bin = bin;
      sm.sel_above = a;
      sm.sel_cnt = cnt;
    }
  }
  __syncthreads();
}

__device__ __forceinline__ void select_bin_mass(RowSmem& sm, uint64_t target) {
  if (threadIdx.x < kWave) {
    const int l = threadIdx.x;
    const int b0 = 255 - 4 * l;
    uint64_t c0 = sm.mhist[b0], c1 = sm.mhist[b0 - 1], c2 = sm.mhist[b0 - 2], c3 = sm.mhist[b0 - 3];
    uint64_t tot = c0 + c1 + c2 + c3;
    uint64_t incl = tot;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      uint64_t n = __shfl_up(incl, o);
      if (l >= o) incl += n;
    }
    uint64_t excl = incl - tot;
    bool hit = (excl < target && target <= incl) || (l == kWave - 1 && target > incl);
    if (hit) {
      uint64_t a = excl;
      int bin;
      uint64_t mass;
      if (a + c0 >= target) { bin = b0; mass = c0; }
      else { a += c0;
        if (a + c1 >= target) { bin = b0 - 1; mass = c1; }
        else { a += c1;
          if (a + c2 >= target) { bin = b0 - 2; mass = c2; }
          else { a += c2; bin = b0 - 3; mass = c3; } } }
      sm.sel_bin = bin;
      sm.sel_above64 = a;
      sm.sel_mass = mass;
      sm.sel_cnt = sm.hist[bin];
    }
  }
  __syncthreads();
}

__device__ __forceinline__ void clear_hists(RowSmem& sm, bool with_mass) {
  if (threadIdx.x < 256) {
    sm.hist[threadIdx.x] = 0;
    if (with_mass) sm.mhist[threadIdx.x] = 0;
  }
  __syncthreads();
}

// ------------------------------------------------------------- row modes ---

enum PMode : int { kPNone = 0, kPTopOnly = 1, kPBoundary = 2 };

struct RowParams {
  bool k_on;     // 1 <= k <= V-1
  uint32_t k;
  int pmode;     // kPNone: no top-p (p absent, or t <= 0); kPTopOnly: t >= 1
  float t;       // 1 - p in fp32
};

template <class DT>
__device__ __forceinline__ RowParams decode_row_params(const typename DT::raw_t* p, const int32_t* k, int b, int V) {
  RowParams rp;
  rp.k_on = false;
  rp.k = 0;
  if (k != nullptr) {
    int32_t kb = k[b];
    if (kb >= 1 && kb <= V - 1) {
      rp.k_on = true;
      rp.k = static_cast<uint32_t>(kb);
    }
  }
  rp.pmode = kPNone;
  rp.t = 0.0f;
  if (p != nullptr) {
    float pb = DT::value(p[b]);
    float t = 1.0f - pb;
    rp.t = t;
    if (t >= 1.0f) rp.pmode = kPTopOnly;
    else if (t > 0.0f) rp.pmode = kPBoundary;
    // t <= 0 (p >= 1) or NaN: no position with positive mass is masked
  }
  return rp;
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
