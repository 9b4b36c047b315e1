// C ABI of libtopktopp: argument checks and dispatch to the HIP launchers.
// The checks follow the order of the aclnn parameter checks described in the
// ApplyTopKTopPWithSorted guide (§5.3): null pointers, then dtype, then shape.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <string>

#include "../../include/topktopp.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;
std::atomic<int> g_policy{tkp::kPlanAuto};

topktopp_status fail(topktopp_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

size_t elem_size(int dtype) { return dtype == TOPKTOPP_F32 ? 4 : 2; }

bool valid_dtype(int dtype) { return dtype == TOPKTOPP_F32 || dtype == TOPKTOPP_F16 || dtype == TOPKTOPP_BF16; }

// [a, a + na) and [b, b + nb) overlap (byte ranges).
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

topktopp_status check_shape(int64_t B, int64_t V) {
  if (B < 0 || V < 0) return fail(TOPKTOPP_ERR_INVALID, "shape [%lld, %lld] has a negative extent", (long long)B, (long long)V);
  if (V > TOPKTOPP_MAX_V)
    return fail(TOPKTOPP_ERR_INVALID, "row length V=%lld exceeds the supported maximum %d", (long long)V, TOPKTOPP_MAX_V);
  if (B > TOPKTOPP_MAX_B)
    return fail(TOPKTOPP_ERR_INVALID, "B=%lld rows exceeds the supported maximum 2^31-1", (long long)B);
  return TOPKTOPP_OK;
}

// Row strides: every operand's rows are at least V elements apart (rows may
// not overlap one another), and small enough for the byte offsets to fit.
topktopp_status check_ld(int64_t ld, int64_t V, const char* name) {
  if (ld < V) return fail(TOPKTOPP_ERR_INVALID, "row stride of %s (%lld) is below V=%lld", name, (long long)ld, (long long)V);
  if (ld > TOPKTOPP_MAX_LD)
    return fail(TOPKTOPP_ERR_INVALID, "row stride of %s (%lld) exceeds the supported maximum", name, (long long)ld);
  return TOPKTOPP_OK;
}

// Bytes from the first element of a strided [B, V] operand to one past its last.
size_t extent(int64_t B, int64_t V, int64_t ld, size_t es) {
  return (static_cast<size_t>(B - 1) * static_cast<size_t>(ld) + static_cast<size_t>(V)) * es;
}

topktopp_status check_launch(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(TOPKTOPP_ERR_RUNTIME, "%s failed: %s", what, hipGetErrorString(e));
  return TOPKTOPP_OK;
}

}  // namespace

extern "C" {

const char* topktopp_last_error(void) { return g_last_error.c_str(); }

int topktopp_set_plan_policy(int policy) {
  if (policy < tkp::kPlanAuto || policy > tkp::kPlanStream) return -1;
  return g_policy.exchange(policy);
}

}  // extern "C"

namespace {

// The entry points without min_p pass has_min_p = false: then p and k may
// not both be NULL, as in the aclnn checks; with it, any one of the three.
topktopp_status check_params(const void* p, const int32_t* k, const void* min_p, bool has_min_p) {
  if (p == nullptr && k == nullptr && min_p == nullptr)
    return has_min_p ? fail(TOPKTOPP_ERR_NULLPTR, "p, k and min_p are all NULL; at least one is required")
                     : fail(TOPKTOPP_ERR_NULLPTR, "p and k are both NULL; at least one is required");
  return TOPKTOPP_OK;
}

topktopp_status apply_impl(const void* logits, int64_t ldx, int dtype, int64_t B, int64_t V, const void* p,
                           const int32_t* k, const void* min_p, bool has_min_p, void* out, int64_t ldo,
                           void* stream) {
  g_last_error.clear();
  if (B >= 0 && V >= 0 && (B == 0 || V == 0)) {  // empty: nothing is read or written, pointers may be NULL
    if (!valid_dtype(dtype)) return fail(TOPKTOPP_ERR_INVALID, "dtype %d is not one of F32, F16, BF16", dtype);
    return TOPKTOPP_OK;
  }
  if (logits == nullptr) return fail(TOPKTOPP_ERR_NULLPTR, "logits is NULL");
  if (out == nullptr) return fail(TOPKTOPP_ERR_NULLPTR, "out is NULL");
  if (topktopp_status s = check_params(p, k, min_p, has_min_p)) return s;
  if (!valid_dtype(dtype)) return fail(TOPKTOPP_ERR_INVALID, "dtype %d is not one of F32, F16, BF16", dtype);
  if (topktopp_status s = check_shape(B, V)) return s;
  if (topktopp_status s = check_ld(ldx, V, "logits")) return s;
  if (topktopp_status s = check_ld(ldo, V, "out")) return s;
  const size_t es = elem_size(dtype);
  const size_t nout = extent(B, V, ldo, es);
  if (overlaps(out, nout, logits, extent(B, V, ldx, es)) || overlaps(out, nout, p, static_cast<size_t>(B) * es) ||
      overlaps(out, nout, k, static_cast<size_t>(B) * 4) || overlaps(out, nout, min_p, static_cast<size_t>(B) * es))
    return fail(TOPKTOPP_ERR_INVALID, "out overlaps an input buffer");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (V == 1)  // a last dimension of 1 is copied through unfiltered
    return check_launch(hipMemcpy2DAsync(out, static_cast<size_t>(ldo) * es, logits, static_cast<size_t>(ldx) * es, es,
                                         static_cast<size_t>(B), hipMemcpyDeviceToDevice, st),
                        "hipMemcpy2DAsync");
  const tkp::RowStrides ld{ldx, ldo, 0, 0};
  return check_launch(tkp::launch_apply(dtype, logits, p, k, min_p, out, B, V, ld, g_policy.load(), st),
                      "filter launch");
}

// Strides of a strided view: in [lo, TOPKTOPP_MAX_LD].
topktopp_status check_stride(int64_t s, int64_t lo, const char* name) {
  if (s < lo || s > TOPKTOPP_MAX_LD)
    return fail(TOPKTOPP_ERR_INVALID, "stride %s=%lld is outside [%lld, 2^31]", name, (long long)s, (long long)lo);
  return TOPKTOPP_OK;
}

// Bytes from the first to one past the last element of a [B, V] view with
// non-negative strides sr (rows) and sc (elements).
size_t span2(int64_t B, int64_t V, int64_t sr, int64_t sc, size_t es) {
  return (static_cast<size_t>(B - 1) * static_cast<size_t>(sr) + static_cast<size_t>(V - 1) * static_cast<size_t>(sc) + 1) *
         es;
}

topktopp_status strided_impl(const void* logits, int64_t xr, int64_t xc, int dtype, int64_t B, int64_t V,
                             const void* p, int64_t ps, const int32_t* k, int64_t ks, const void* min_p, int64_t ms,
                             void* out, int64_t orr, int64_t oc, void* stream) {
  g_last_error.clear();
  if (B >= 0 && V >= 0 && (B == 0 || V == 0)) {  // empty: nothing is read or written, pointers may be NULL
    if (!valid_dtype(dtype)) return fail(TOPKTOPP_ERR_INVALID, "dtype %d is not one of F32, F16, BF16", dtype);
    return TOPKTOPP_OK;
  }
  if (logits == nullptr) return fail(TOPKTOPP_ERR_NULLPTR, "logits is NULL");
  if (out == nullptr) return fail(TOPKTOPP_ERR_NULLPTR, "out is NULL");
  if (topktopp_status s = check_params(p, k, min_p, true)) return s;
  if (!valid_dtype(dtype)) return fail(TOPKTOPP_ERR_INVALID, "dtype %d is not one of F32, F16, BF16", dtype);
  if (topktopp_status s = check_shape(B, V)) return s;
  // a stride along an extent of 1 plays no part: take it as 0 (inputs) or 1 (out)
  if (B == 1) xr = ps = ks = ms = 0, orr = 1;
  if (V == 1) xc = 0, oc = 1;
  if (p == nullptr) ps = 0;
  if (k == nullptr) ks = 0;
  if (min_p == nullptr) ms = 0;
  if (topktopp_status s = check_stride(xr, 0, "logits_row_stride")) return s;
  if (topktopp_status s = check_stride(xc, 0, "logits_col_stride")) return s;
  if (topktopp_status s = check_stride(ps, 0, "p_stride")) return s;
  if (topktopp_status s = check_stride(ks, 0, "k_stride")) return s;
  if (topktopp_status s = check_stride(ms, 0, "min_p_stride")) return s;
  if (topktopp_status s = check_stride(orr, 1, "out_row_stride")) return s;
  if (topktopp_status s = check_stride(oc, 1, "out_col_stride")) return s;
  if (!(orr >= V * oc || oc >= B * orr))
    return fail(TOPKTOPP_ERR_INVALID,
                "out strides (%lld, %lld) may map two positions of [%lld, %lld] to one element", (long long)orr,
                (long long)oc, (long long)B, (long long)V);
  const size_t es = elem_size(dtype);
  const size_t nout = span2(B, V, orr, oc, es);
  if (overlaps(out, nout, logits, span2(B, V, xr, xc, es)) || overlaps(out, nout, p, span2(B, 1, ps, 0, es)) ||
      overlaps(out, nout, k, span2(B, 1, ks, 0, 4)) || overlaps(out, nout, min_p, span2(B, 1, ms, 0, es)))
    return fail(TOPKTOPP_ERR_INVALID, "out overlaps an input buffer");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (V == 1)  // a last dimension of 1 is copied through unfiltered (row strides of any value, 0 included)
    return check_launch(tkp::launch_copy_column(logits, xr, out, orr, B, static_cast<int>(es), st), "copy launch");
  // contiguous rows and dense parameters: the row-strided path
  const bool dense_params = (p == nullptr || B == 1 || ps == 1) && (k == nullptr || B == 1 || ks == 1) &&
                            (min_p == nullptr || B == 1 || ms == 1);
  if (xc == 1 && oc == 1 && dense_params && (B == 1 || (xr >= V && orr >= V)))
    return apply_impl(logits, B == 1 ? V : xr, dtype, B, V, p, k, min_p, true, out, B == 1 ? V : orr, stream);
  tkp::RowStrides ld{xr, orr, 0, 0};
  ld.elementwise = true;
  ld.xc = xc;
  ld.oc = oc;
  ld.pc = ps;
  ld.kc = ks;
  ld.mc = ms;
  return check_launch(tkp::launch_apply(dtype, logits, p, k, min_p, out, B, V, ld, g_policy.load(), st),
                      "filter launch");
}

topktopp_status with_sorted_impl(const void* sorted_value, int64_t lds, const int32_t* sorted_indices, int64_t ldi,
                                 int dtype, int64_t B, int64_t V, const void* p, const int32_t* k,
                                 const void* min_p, bool has_min_p, const void* logits, int64_t ldx, void* out,
                                 int64_t ldo, void* stream) {
  g_last_error.clear();
  if (B >= 0 && V >= 0 && (B == 0 || V == 0)) {  // empty: nothing is read or written, pointers may be NULL
    if (!valid_dtype(dtype)) return fail(TOPKTOPP_ERR_INVALID, "dtype %d is not one of F32, F16, BF16", dtype);
    return TOPKTOPP_OK;
  }
  if (sorted_value == nullptr) return fail(TOPKTOPP_ERR_NULLPTR, "sorted_value is NULL");
  if (sorted_indices == nullptr) return fail(TOPKTOPP_ERR_NULLPTR, "sorted_indices is NULL");
  if (out == nullptr) return fail(TOPKTOPP_ERR_NULLPTR, "out is NULL");
  if (topktopp_status s = check_params(p, k, min_p, has_min_p)) return s;
  if (!valid_dtype(dtype)) return fail(TOPKTOPP_ERR_INVALID, "dtype %d is not one of F32, F16, BF16", dtype);
  if (topktopp_status s = check_shape(B, V)) return s;
  if (topktopp_status s = check_ld(lds, V, "sorted_value")) return s;
  if (topktopp_status s = check_ld(ldi, V, "sorted_indices")) return s;
  if (logits != nullptr)
    if (topktopp_status s = check_ld(ldx, V, "logits")) return s;
  if (topktopp_status s = check_ld(ldo, V, "out")) return s;
  const size_t es = elem_size(dtype);
  const size_t nout = extent(B, V, ldo, es);
  if (overlaps(out, nout, sorted_value, extent(B, V, lds, es)) ||
      overlaps(out, nout, sorted_indices, extent(B, V, ldi, 4)) ||
      (logits != nullptr && overlaps(out, nout, logits, extent(B, V, ldx, es))) ||
      overlaps(out, nout, p, static_cast<size_t>(B) * es) || overlaps(out, nout, k, static_cast<size_t>(B) * 4) ||
      overlaps(out, nout, min_p, static_cast<size_t>(B) * es))
    return fail(TOPKTOPP_ERR_INVALID, "out overlaps an input buffer");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (V == 1) {  // the single element is always kept; sorted_indices is 0
    const void* src = logits != nullptr ? logits : sorted_value;
    const int64_t lsrc = logits != nullptr ? ldx : lds;
    return check_launch(hipMemcpy2DAsync(out, static_cast<size_t>(ldo) * es, src, static_cast<size_t>(lsrc) * es, es,
                                         static_cast<size_t>(B), hipMemcpyDeviceToDevice, st),
                        "hipMemcpy2DAsync");
  }
  const tkp::RowStrides ld{logits != nullptr ? ldx : V, ldo, lds, ldi};
  return check_launch(
      tkp::launch_with_sorted(dtype, sorted_value, sorted_indices, p, k, min_p, logits, out, B, V, ld, st),
      "filter launch");
}

topktopp_status sample_impl(const void* logits, int dtype, int64_t B, int64_t V, const void* p, const int32_t* k,
                            const void* min_p, const float* q, float eps, void* out, int32_t* selected,
                            void* stream) {
  g_last_error.clear();
  if (B >= 0 && V >= 0 && (B == 0 || V == 0)) {  // empty: nothing is read or written, pointers may be NULL
    if (!valid_dtype(dtype)) return fail(TOPKTOPP_ERR_INVALID, "dtype %d is not one of F32, F16, BF16", dtype);
    return TOPKTOPP_OK;
  }
  if (logits == nullptr) return fail(TOPKTOPP_ERR_NULLPTR, "logits is NULL");
  if (selected == nullptr) return fail(TOPKTOPP_ERR_NULLPTR, "selected is NULL");
  if (!valid_dtype(dtype)) return fail(TOPKTOPP_ERR_INVALID, "dtype %d is not one of F32, F16, BF16", dtype);
  if (topktopp_status s = check_shape(B, V)) return s;
  if (!(eps >= 0.0f) || eps > 3.0e38f) return fail(TOPKTOPP_ERR_INVALID, "eps must be finite and >= 0");
  const size_t es = elem_size(dtype);
  const size_t nx = static_cast<size_t>(B) * static_cast<size_t>(V) * es;
  const size_t nq = static_cast<size_t>(B) * static_cast<size_t>(V) * 4;
  const size_t nsel = static_cast<size_t>(B) * 4;
  if (out != nullptr &&
      (overlaps(out, nx, logits, nx) || overlaps(out, nx, p, static_cast<size_t>(B) * es) ||
       overlaps(out, nx, k, static_cast<size_t>(B) * 4) || overlaps(out, nx, min_p, static_cast<size_t>(B) * es) ||
       overlaps(out, nx, q, nq) || overlaps(out, nx, selected, nsel)))
    return fail(TOPKTOPP_ERR_INVALID, "out overlaps another buffer");
  if (overlaps(selected, nsel, logits, nx) || overlaps(selected, nsel, p, static_cast<size_t>(B) * es) ||
      overlaps(selected, nsel, k, static_cast<size_t>(B) * 4) ||
      overlaps(selected, nsel, min_p, static_cast<size_t>(B) * es) || overlaps(selected, nsel, q, nq))
    return fail(TOPKTOPP_ERR_INVALID, "selected overlaps an input buffer");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (V == 1) {  // one element per row: it is kept and it is the pick
    if (out != nullptr)
      if (topktopp_status s = check_launch(hipMemcpyAsync(out, logits, nx, hipMemcpyDeviceToDevice, st), "hipMemcpyAsync"))
        return s;
    return check_launch(tkp::launch_fill_zero_i32(selected, B, st), "fill launch");
  }
  const tkp::RowStrides ld{V, V, 0, 0};
  const tkp::SampleArgs sa{q, V, eps, selected, nullptr, nullptr, nullptr, 0};
  return check_launch(tkp::launch_sample(dtype, logits, p, k, min_p, out, B, V, ld, g_policy.load(), st, sa),
                      "sample launch");
}

topktopp_status survivors_impl(const void* logits, int dtype, int64_t B, int64_t V, const void* p, const int32_t* k,
                               const void* min_p, int64_t cap, float* probs, int32_t* indices, int32_t* counts,
                               void* stream) {
  g_last_error.clear();
  if (B >= 0 && V >= 0 && (B == 0 || V == 0)) {  // empty: nothing is read or written, pointers may be NULL
    if (!valid_dtype(dtype)) return fail(TOPKTOPP_ERR_INVALID, "dtype %d is not one of F32, F16, BF16", dtype);
    return TOPKTOPP_OK;
  }
  if (logits == nullptr) return fail(TOPKTOPP_ERR_NULLPTR, "logits is NULL");
  if (indices == nullptr) return fail(TOPKTOPP_ERR_NULLPTR, "indices is NULL");
  if (counts == nullptr) return fail(TOPKTOPP_ERR_NULLPTR, "counts is NULL");
  if (!valid_dtype(dtype)) return fail(TOPKTOPP_ERR_INVALID, "dtype %d is not one of F32, F16, BF16", dtype);
  if (topktopp_status s = check_shape(B, V)) return s;
  if (cap < 1 || cap > TOPKTOPP_MAX_V) return fail(TOPKTOPP_ERR_INVALID, "cap=%lld is outside [1, 2^20]", (long long)cap);
  const size_t es = elem_size(dtype);
  const size_t nx = static_cast<size_t>(B) * static_cast<size_t>(V) * es;
  const size_t ncap = static_cast<size_t>(B) * static_cast<size_t>(cap) * 4;
  const void* inputs[4] = {logits, p, k, min_p};
  const size_t sizes[4] = {nx, static_cast<size_t>(B) * es, static_cast<size_t>(B) * 4, static_cast<size_t>(B) * es};
  const void* outs[3] = {probs, indices, counts};
  const size_t osz[3] = {ncap, ncap, static_cast<size_t>(B) * 4};
  for (int o = 0; o < 3; ++o) {
    for (int i = 0; i < 4; ++i)
      if (overlaps(outs[o], osz[o], inputs[i], sizes[i])) return fail(TOPKTOPP_ERR_INVALID, "an output overlaps an input buffer");
    for (int o2 = o + 1; o2 < 3; ++o2)
      if (overlaps(outs[o], osz[o], outs[o2], osz[o2])) return fail(TOPKTOPP_ERR_INVALID, "two outputs overlap");
  }
  if (V == 1) return check_launch(tkp::launch_survivors_single(probs, indices, counts, B, cap,
                                                              static_cast<hipStream_t>(stream)),
                                  "survivors launch");
  const tkp::RowStrides ld{V, V, 0, 0};
  const tkp::SampleArgs sa{nullptr, V, 0.0f, nullptr, probs, indices, counts, cap};
  return check_launch(tkp::launch_sample(dtype, logits, p, k, min_p, nullptr, B, V, ld, g_policy.load(),
                                         static_cast<hipStream_t>(stream), sa),
                      "survivors launch");
}

}  // namespace

extern "C" {

topktopp_status sample_top_k_top_p(const void* logits, topktopp_dtype dtype, int64_t B, int64_t V, const void* p,
                                   const int32_t* k, const void* min_p, const float* q, float eps, void* out,
                                   int32_t* selected, void* stream) {
  return sample_impl(logits, dtype, B, V, p, k, min_p, q, eps, out, selected, stream);
}

topktopp_status top_k_top_p_sorted_survivors(const void* logits, topktopp_dtype dtype, int64_t B, int64_t V, const void* p,
                                             const int32_t* k, const void* min_p, int64_t cap, float* probs,
                                             int32_t* indices, int32_t* counts, void* stream) {
  return survivors_impl(logits, dtype, B, V, p, k, min_p, cap, probs, indices, counts, stream);
}

topktopp_status apply_top_k_top_p(const void* logits, topktopp_dtype dtype, int64_t B, int64_t V, const void* p,
                                  const int32_t* k, void* out, void* stream) {
  return apply_impl(logits, V, dtype, B, V, p, k, nullptr, false, out, V, stream);
}

topktopp_status apply_top_k_top_p_min_p(const void* logits, topktopp_dtype dtype, int64_t B, int64_t V, const void* p,
                                        const int32_t* k, const void* min_p, void* out, void* stream) {
  return apply_impl(logits, V, dtype, B, V, p, k, min_p, true, out, V, stream);
}

topktopp_status apply_top_k_top_p_ex(const void* logits, int64_t ld_logits, topktopp_dtype dtype, int64_t B, int64_t V,
                                     const void* p, const int32_t* k, const void* min_p, void* out, int64_t ld_out,
                                     void* stream) {
  return apply_impl(logits, ld_logits, dtype, B, V, p, k, min_p, true, out, ld_out, stream);
}

topktopp_status apply_top_k_top_p_strided(const void* logits, int64_t logits_row_stride, int64_t logits_col_stride,
                                          topktopp_dtype dtype, int64_t B, int64_t V, const void* p, int64_t p_stride,
                                          const int32_t* k, int64_t k_stride, const void* min_p,
                                          int64_t min_p_stride, void* out, int64_t out_row_stride,
                                          int64_t out_col_stride, void* stream) {
  return strided_impl(logits, logits_row_stride, logits_col_stride, dtype, B, V, p, p_stride, k, k_stride, min_p,
                      min_p_stride, out, out_row_stride, out_col_stride, stream);
}

topktopp_status apply_top_k_top_p_with_sorted(const void* sorted_value, const int32_t* sorted_indices, topktopp_dtype dtype,
                                              int64_t B, int64_t V, const void* p, const int32_t* k,
                                              const void* logits, void* out, void* stream) {
  return with_sorted_impl(sorted_value, V, sorted_indices, V, dtype, B, V, p, k, nullptr, false, logits, V, out, V,
                          stream);
}

topktopp_status apply_top_k_top_p_min_p_with_sorted(const void* sorted_value, const int32_t* sorted_indices,
                                                    topktopp_dtype dtype, int64_t B, int64_t V, const void* p,
                                                    const int32_t* k, const void* min_p, const void* logits,
                                                    void* out, void* stream) {
  return with_sorted_impl(sorted_value, V, sorted_indices, V, dtype, B, V, p, k, min_p, true, logits, V, out, V,
                          stream);
}

topktopp_status apply_top_k_top_p_with_sorted_ex(const void* sorted_value, int64_t ld_sorted_value,
                                                 const int32_t* sorted_indices, int64_t ld_sorted_indices, topktopp_dtype dtype,
                                                 int64_t B, int64_t V, const void* p, const int32_t* k,
                                                 const void* min_p, const void* logits, int64_t ld_logits, void* out,
                                                 int64_t ld_out, void* stream) {
  return with_sorted_impl(sorted_value, ld_sorted_value, sorted_indices, ld_sorted_indices, dtype, B, V, p, k, min_p,
                          true, logits, ld_logits, out, ld_out, stream);
}

}  // extern "C"
