// CPU oracle for the top-k / top-p logits filter: plain, single-threaded C++17.
//
// TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU baseline of
// the benchmark load this library (through oracle/topktopp_oracle.py). The HIP
// path never links or calls it, and the two share no code: not the key
// transform, not the dtype conversions, not the -inf constants, not the
// arithmetic.
//
// Sources. "AKP" is the CANN ops-nn page "ApplyTopKTopPWithSorted 的
// top-k/top-p 采样过滤原理与 aclnn 调用指南", the filter's own description;
// "TKS" is Ascend's "aclnnTopKTopPSampleV2" page (the min-p stage and the
// sampling stage after the filter).
//
// What a row computes (AKP §2, steps 1-8). The row is ranked by a stable
// ascending sort: rank j holds the j-th smallest value, equal values in index
// order (AKP §6.1: the aclnn entry sorts ascending and stable). Each stage then
// decides, rank by rank, whether the position at that rank survives:
//   * top-k (steps 1-3): the threshold is the value at rank V - k, the k-th
//     largest; a rank survives iff its value is not strictly below it. k <= 0
//     or k >= V disables the stage (AKP §4, §5.2 parameter table);
//   * top-p (steps 4-7): the probabilities are a softmax over the top-k
//     survivors, the cumulative probability of rank j is the sum over ranks
//     0..j (the mass at or below it, smallest first); a rank survives iff that
//     sum, rounded to fp32, is above 1 - p, and the top rank always survives;
//   * min-p (TKS "minP sampling"): a rank survives iff its step-4 probability
//     is not below the largest probability left after top-p times min_p;
//     min_p >= 1 keeps only the top rank, min_p <= 0 skips the stage.
// The output (step 8) is assembled from these decisions in the original
// vocabulary order: a surviving position holds its input bits, every other
// position the dtype's -inf.
//
// Readings where the pages are garbled or silent:
//   * the comparison operators were lost in the page text: top-k masks values
//     strictly below the threshold and top-p masks cumulative sums <= 1 - p,
//     as the prose of steps 2 and 6 says;
//   * step 8 puts each ranked value back at its original index (the golden's
//     scatter; the gather as typeset would not restore the original order);
//   * values compare as IEEE floats, so -0.0 and +0.0 are equal and keep index
//     order; kept values are copied as bits, so a kept -0.0 stays -0.0;
//   * the softmax and the cumulative sum are carried out in double and the
//     cumulative sum is rounded to fp32 (the golden's tensor type) only for
//     the comparison with 1 - p, which keeps the oracle's own rounding far
//     below the 1e-5 band the GPU comparison allows;
//   * 1 - p is an fp32 subtraction of p widened exactly (t_reading 0); the
//     other plausible reading, 1 - p rounded to p's own dtype (t_reading 1),
//     is kept to count where the two disagree;
//   * pre-sorted input: ranks are the given positions, ties included; with
//     logits, kept values are read from the logits in original order (AKP §3).
// Sampling (TKS "Subsequent processing"): descending rank d is ascending rank
// V - 1 - d, so equal values take the higher index first. The argmax ("None"
// mode) is the top rank; QSample is the first maximum over d of
// prob(d) / (q[d] + eps), masked ranks scoring 0. The sorted-survivors output
// (TKS "Intermediate result output") lists the survivors by descending rank
// with their step-4 probabilities.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <numeric>
#include <vector>

namespace {

enum Dtype : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

// ---------------------------------------------------------------- storage ---

uint32_t load_bits(const void* base, int dtype, int64_t i) {
  if (dtype == kF32) return static_cast<const uint32_t*>(base)[i];
  return static_cast<const uint16_t*>(base)[i];
}

void store_bits(void* base, int dtype, int64_t i, uint32_t bits) {
  if (dtype == kF32)
    static_cast<uint32_t*>(base)[i] = bits;
  else
    static_cast<uint16_t*>(base)[i] = static_cast<uint16_t>(bits);
}

float f32_from_bits(uint32_t u) {
  float f;
  std::memcpy(&f, &u, sizeof f);
  return f;
}

uint32_t bits_from_f32(float f) {
  uint32_t u;
  std::memcpy(&u, &f, sizeof u);
  return u;
}

// IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
double f16_value(uint32_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 31;
  const int f = h & 1023;
  double v;
  if (e == 0)
    v = std::ldexp(static_cast<double>(f), -24);  // subnormal: f * 2^-24
  else if (e == 31)
    v = f == 0 ? std::numeric_limits<double>::infinity() : std::numeric_limits<double>::quiet_NaN();
  else
    v = std::ldexp(static_cast<double>(1024 + f), e - 25);  // (1 + f/1024) * 2^(e-15)
  return sign ? -v : v;
}

// Exact value of a stored element (every fp32/fp16/bf16 value is a double).
double widen(uint32_t bits, int dtype) {
  if (dtype == kF32) return static_cast<double>(f32_from_bits(bits));
  if (dtype == kBF16) return static_cast<double>(f32_from_bits(bits << 16));  // bf16: the top half of an fp32
  return f16_value(bits);
}

// The dtype's -inf (AKP §6.3 lists the kernel constants).
uint32_t neg_inf_bits(int dtype) {
  if (dtype == kF32) return 0xFF800000u;
  if (dtype == kF16) return 0xFC00u;
  return 0xFF80u;
}

// A finite float rounded to the nearest value of the dtype, ties to even.
float round_to_dtype(float v, int dtype) {
  if (dtype == kF32) return v;
  if (dtype == kBF16) {
    // keep the top 16 bits of the fp32 pattern, rounding on the 16 dropped
    const uint32_t u = bits_from_f32(v);
    const uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) & 0xFFFF0000u;
    return f32_from_bits(r);
  }
  // fp16: 10 fraction bits; the spacing is 2^(e - 10) for |v| in [2^e, 2^(e+1)),
  // e >= -14 (below that the subnormal spacing 2^-24)
  const double d = static_cast<double>(v);
  if (d == 0.0) return v;
  int e = static_cast<int>(std::floor(std::log2(std::fabs(d))));
  if (std::ldexp(1.0, e) > std::fabs(d)) --e;  // guard log2 rounding
  if (std::ldexp(1.0, e + 1) <= std::fabs(d)) ++e;
  if (e < -14) e = -14;
  const double quantum = std::ldexp(1.0, e - 10);
  const double q = std::nearbyint(d / quantum) * quantum;  // default rounding: ties to even
  if (std::fabs(q) > 65504.0) return d > 0 ? std::numeric_limits<float>::infinity() : -std::numeric_limits<float>::infinity();
  return static_cast<float>(q);
}

// t = 1 - p as step 6 compares it.
float one_minus_p(uint32_t p_bits, int dtype, int t_reading) {
  const float p = static_cast<float>(widen(p_bits, dtype));  // exact
  const float t = 1.0f - p;                                // fp32 subtraction
  return t_reading == 1 ? round_to_dtype(t, dtype) : t;
}

// ------------------------------------------------------------- one row -----

// Per-row parameters; absent ones have has_* false.
struct Params {
  bool has_k = false, has_p = false, has_min_p = false;
  int64_t k = 0;
  uint32_t p_bits = 0, min_p_bits = 0;
};

// What the stages decided, by ascending rank (all vectors of length V).
struct Decisions {
  std::vector<uint8_t> masked_k, masked_p, masked_m;
  std::vector<double> prob;     // step-4 probability of each rank
  std::vector<float> cum32;     // cumulative probability at or below each rank, rounded to fp32
  std::vector<double> ratio_m;  // probability over the min-p threshold (0 < min_p < 1 only)
  float t = 0.0f;
  bool p_active = false, ratio_valid = false;
  bool survives(int64_t j) const { return !masked_k[j] && !masked_p[j] && !masked_m[j]; }
};

// The stages of AKP §2 (and TKS min-p) on one row ranked ascending: s[j] is
// the value at rank j.
Decisions decide(const std::vector<double>& s, const Params& prm, int dtype, int t_reading) {
  const int64_t V = static_cast<int64_t>(s.size());
  Decisions d;
  d.masked_k.assign(V, 0);
  d.masked_p.assign(V, 0);
  d.masked_m.assign(V, 0);
  // steps 1-3: the k-th largest value is the one at rank V - k
  if (prm.has_k && prm.k >= 1 && prm.k <= V - 1) {
    const double kth = s[V - prm.k];
    for (int64_t j = 0; j < V; ++j) d.masked_k[j] = s[j] < kth ? 1 : 0;
  }
  // step 4: softmax over the top-k survivors; the top rank holds the maximum
  const double m = s[V - 1];
  std::vector<double> e(V, 0.0);
  double Z = 0.0;
  for (int64_t j = 0; j < V; ++j) {  // summed from the smallest up
    e[j] = d.masked_k[j] ? 0.0 : std::exp(s[j] - m);
    Z += e[j];
  }
  d.prob.assign(V, 0.0);
  for (int64_t j = 0; j < V; ++j) d.prob[j] = e[j] / Z;
  // step 5: the cumulative probability at or below each rank, smallest first
  d.cum32.assign(V, 0.0f);
  double c = 0.0;
  for (int64_t j = 0; j < V; ++j) {
    c += d.prob[j];
    d.cum32[j] = static_cast<float>(c);
  }
  // steps 6-7: ranks whose cumulative probability is <= 1 - p are masked,
  // except the top rank
  if (prm.has_p) {
    d.p_active = true;
    d.t = one_minus_p(prm.p_bits, dtype, t_reading);
    for (int64_t j = 0; j < V - 1; ++j) d.masked_p[j] = d.cum32[j] <= d.t ? 1 : 0;
  }
  // min-p: the largest probability left after top-p is the top rank's
  if (prm.has_min_p) {
    const double mp = widen(prm.min_p_bits, dtype);
    if (mp >= 1.0) {
      for (int64_t j = 0; j < V - 1; ++j) d.masked_m[j] = 1;  // one token: the top rank
    } else if (mp > 0.0) {
      const double thr = d.prob[V - 1] * mp;
      d.ratio_m.assign(V, 0.0);
      d.ratio_valid = true;
      for (int64_t j = 0; j < V; ++j) {
        d.ratio_m[j] = d.prob[j] / thr;
        // positions top-p masked are set aside (TKS applies min-p to what top-p left)
        d.masked_m[j] = (d.masked_p[j] || d.prob[j] < thr) ? 1 : 0;
      }
    }
  }
  return d;
}

// Ascending stable ranking of a row: order[j] is the original index at rank j.
std::vector<int64_t> stable_ranking(const std::vector<double>& x) {
  std::vector<int64_t> order(x.size());
  std::iota(order.begin(), order.end(), int64_t{0});
  std::stable_sort(order.begin(), order.end(), [&](int64_t a, int64_t b) { return x[a] < x[b]; });
  return order;
}

}  // namespace

// ------------------------------------------------------------- C ABI -------
//
// Arrays are row-major; bits are uint32 (fp32) or uint16 (fp16, bf16). Trace
// arrays are indexed by [row, ascending rank] and may each be NULL; per-row
// flags say which are meaningful.

extern "C" {

struct OracleTrace {
  int64_t* order;      // [B, V] original index at each rank
  uint8_t* masked_k;   // [B, V]
  uint8_t* masked_p;   // [B, V]
  uint8_t* masked_m;   // [B, V]
  float* cum32;        // [B, V] cumulative probability, fp32
  double* ratio_m;     // [B, V] probability over the min-p threshold
  double* prob;        // [B, V] step-4 probability
  float* t;            // [B] 1 - p as compared
  uint8_t* p_active;   // [B] top-p ran (cum32 and t meaningful)
  uint8_t* ratio_valid;  // [B] ratio_m meaningful
};

float oracle_one_minus_p(uint32_t p_bits, int dtype, int t_reading) { return one_minus_p(p_bits, dtype, t_reading); }

double oracle_widen(uint32_t bits, int dtype) { return widen(bits, dtype); }

}  // extern "C"

namespace {

Params row_params(int64_t b, const void* p, const int32_t* k, const void* min_p, int dtype) {
  Params prm;
  if (k != nullptr) {
    prm.has_k = true;
    prm.k = k[b];
  }
  if (p != nullptr) {
    prm.has_p = true;
    prm.p_bits = load_bits(p, dtype, b);
  }
  if (min_p != nullptr) {
    prm.has_min_p = true;
    prm.min_p_bits = load_bits(min_p, dtype, b);
  }
  return prm;
}

void record(OracleTrace* tr, int64_t b, int64_t V, const std::vector<int64_t>& order, const Decisions& d) {
  if (tr == nullptr) return;
  const int64_t o = b * V;
  for (int64_t j = 0; j < V; ++j) {
    if (tr->order) tr->order[o + j] = order[j];
    if (tr->masked_k) tr->masked_k[o + j] = d.masked_k[j];
    if (tr->masked_p) tr->masked_p[o + j] = d.masked_p[j];
    if (tr->masked_m) tr->masked_m[o + j] = d.masked_m[j];
    if (tr->cum32) tr->cum32[o + j] = d.cum32[j];
    if (tr->prob) tr->prob[o + j] = d.prob[j];
    if (tr->ratio_m) tr->ratio_m[o + j] = d.ratio_valid ? d.ratio_m[j] : 0.0;
  }
  if (tr->t) tr->t[b] = d.t;
  if (tr->p_active) tr->p_active[b] = d.p_active ? 1 : 0;
  if (tr->ratio_valid) tr->ratio_valid[b] = d.ratio_valid ? 1 : 0;
}

// A row of one element is passed through (AKP §6.1); its trace is trivial.
Decisions single(int64_t V) {
  Decisions d;
  d.masked_k.assign(V, 0);
  d.masked_p.assign(V, 0);
  d.masked_m.assign(V, 0);
  d.prob.assign(V, 1.0);
  d.cum32.assign(V, 1.0f);
  return d;
}

// One row of the sorting entry: ranking, decisions, trace. `x` receives the
// row's values in original order.
Decisions rank_and_decide(const void* logits, int dtype, int64_t b, int64_t V, const Params& prm, int t_reading,
                          std::vector<double>& x, std::vector<int64_t>& order) {
  x.resize(V);
  for (int64_t v = 0; v < V; ++v) x[v] = widen(load_bits(logits, dtype, b * V + v), dtype);
  order = stable_ranking(x);
  if (V == 1) return single(V);
  std::vector<double> s(V);
  for (int64_t j = 0; j < V; ++j) s[j] = x[order[j]];
  return decide(s, prm, dtype, t_reading);
}

// Step 8 for raw logits: each original position takes its input bits when
// the rank it holds survives, and the dtype's -inf otherwise.
void write_row(const void* logits, int dtype, int64_t b, int64_t V, const std::vector<int64_t>& order,
               const Decisions& d, void* out, std::vector<int64_t>& rank) {
  for (int64_t j = 0; j < V; ++j) rank[order[j]] = j;
  for (int64_t v = 0; v < V; ++v) {
    const uint32_t bits = load_bits(logits, dtype, b * V + v);
    store_bits(out, dtype, b * V + v, d.survives(rank[v]) ? bits : neg_inf_bits(dtype));
  }
}

}  // namespace

extern "C" {

// The sorting entry (AKP §5, §6.1): rank each row, decide, write out.
int oracle_apply(const void* logits, int dtype, int64_t B, int64_t V, const void* p, const int32_t* k,
                 const void* min_p, int t_reading, void* out, OracleTrace* tr) {
  std::vector<double> x;
  std::vector<int64_t> order;
  std::vector<int64_t> rank(V);
  for (int64_t b = 0; b < B; ++b) {
    const Params prm = row_params(b, p, k, min_p, dtype);
    const Decisions d = rank_and_decide(logits, dtype, b, V, prm, t_reading, x, order);
    write_row(logits, dtype, b, V, order, d, out, rank);
    record(tr, b, V, order, d);
  }
  return 0;
}

// The pre-sorted operator (AKP §1, §3): ranks are the given positions. With
// logits, a surviving original position holds its logits bits; without, each
// ranked value goes back to its original index.
int oracle_with_sorted(const void* sorted_value, const int64_t* sorted_indices, int dtype, int64_t B, int64_t V,
                       const void* p, const int32_t* k, const void* min_p, const void* logits, int t_reading,
                       void* out, OracleTrace* tr) {
  std::vector<double> s(V);
  std::vector<int64_t> order(V);
  for (int64_t b = 0; b < B; ++b) {
    const Params prm = row_params(b, p, k, min_p, dtype);
    for (int64_t j = 0; j < V; ++j) {
      s[j] = widen(load_bits(sorted_value, dtype, b * V + j), dtype);
      order[j] = sorted_indices[b * V + j];
    }
    const Decisions d = V == 1 ? single(V) : decide(s, prm, dtype, t_reading);
    for (int64_t j = 0; j < V; ++j) {
      const int64_t v = order[j];
      uint32_t bits = neg_inf_bits(dtype);
      if (d.survives(j)) bits = load_bits(logits != nullptr ? logits : sorted_value, dtype, b * V + (logits != nullptr ? v : j));
      store_bits(out, dtype, b * V + v, bits);
    }
    record(tr, b, V, order, d);
  }
  return 0;
}

// The filter followed by TKS's sampling stage. q [B, V] (descending ranks) or
// NULL for the argmax. scores / raw_scores [B, V] (nullable, QSample only): by
// descending rank, prob / (q + eps) where the rank survives (0 elsewhere), and
// the same before the top-p and min-p masks (0 only where top-k masks).
int oracle_sample(const void* logits, int dtype, int64_t B, int64_t V, const void* p, const int32_t* k,
                  const void* min_p, const double* q, double eps, int t_reading, int64_t* selected, double* scores,
                  double* raw_scores, void* out, OracleTrace* tr) {
  std::vector<double> x;
  std::vector<int64_t> order;
  std::vector<int64_t> rank(V);
  for (int64_t b = 0; b < B; ++b) {
    const Params prm = row_params(b, p, k, min_p, dtype);
    const Decisions d = rank_and_decide(logits, dtype, b, V, prm, t_reading, x, order);
    write_row(logits, dtype, b, V, order, d, out, rank);
    record(tr, b, V, order, d);
    if (q == nullptr || V == 1) {
      selected[b] = order[V - 1];  // the first maximum of probs: the top rank
      continue;
    }
    // the first maximum over descending ranks; a NaN score, as in a plain
    // argmax over floats, counts as the largest and the first one wins
    int64_t best_d = -1;
    double best = 0.0;
    bool best_nan = false;
    for (int64_t dd = 0; dd < V; ++dd) {
      const int64_t j = V - 1 - dd;
      const double denom = q[b * V + dd] + eps;
      const double raw = d.masked_k[j] ? 0.0 : d.prob[j] / denom;
      const double sc = d.survives(j) ? d.prob[j] / denom : 0.0;
      if (scores) scores[b * V + dd] = sc;
      if (raw_scores) raw_scores[b * V + dd] = raw;
      if (best_nan) continue;
      if (std::isnan(sc)) {
        best_nan = true;
        best_d = dd;
      } else if (best_d < 0 || sc > best) {
        best = sc;
        best_d = dd;
      }
    }
    selected[b] = order[V - 1 - best_d];
  }
  return 0;
}

// TKS's intermediate output cut to the survivors: for descending rank
// d < min(n, cap), the step-4 probability and the original index; later
// entries hold 0 and -1; counts[b] = n.
int oracle_survivors(const void* logits, int dtype, int64_t B, int64_t V, const void* p, const int32_t* k,
                     const void* min_p, int64_t cap, int t_reading, double* probs, int64_t* indices,
                     int64_t* counts, void* out, OracleTrace* tr) {
  std::vector<double> x;
  std::vector<int64_t> order;
  std::vector<int64_t> rank(V);
  for (int64_t b = 0; b < B; ++b) {
    const Params prm = row_params(b, p, k, min_p, dtype);
    const Decisions d = rank_and_decide(logits, dtype, b, V, prm, t_reading, x, order);
    write_row(logits, dtype, b, V, order, d, out, rank);
    record(tr, b, V, order, d);
    int64_t n = 0;
    for (int64_t dd = 0; dd < V; ++dd) {
      const int64_t j = V - 1 - dd;
      if (!d.survives(j)) continue;  // the survivors are the top ranks
      if (n < cap) {
        probs[b * cap + n] = d.prob[j];
        indices[b * cap + n] = order[j];
      }
      ++n;
    }
    for (int64_t r = n; r < cap; ++r) {
      probs[b * cap + r] = 0.0;
      indices[b * cap + r] = -1;
    }
    counts[b] = n;
  }
  return 0;
}

}  // extern "C"
