// Internal launchers behind the C ABI. Each enqueues on `stream` and returns
// the HIP status of the launch. Shapes are already validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tkp {

// 0: candidate plan, row in registers when it fits; 1: multi-pass plan only,
// row re-read from global memory; 2: candidate plan with the row re-read from
// global memory even when it would fit in registers.
enum PlanPolicy : int { kPlanAuto = 0, kPlanGeneral = 1, kPlanStream = 2 };

// Elements between the starts of consecutive rows of each [B, V] operand
// (each >= V; V when the operand is dense).
struct RowStrides {
  int64_t x;   // logits
  int64_t o;   // out
  int64_t sv;  // sorted_value
  int64_t si;  // sorted_indices
};

hipError_t launch_apply_f32(const void* logits, const void* p, const int32_t* k, const void* min_p, void* out,
                          int64_t B, int64_t V, RowStrides ld, int policy, hipStream_t stream);
hipError_t launch_apply_f16(const void* logits, const void* p, const int32_t* k, const void* min_p, void* out,
                          int64_t B, int64_t V, RowStrides ld, int policy, hipStream_t stream);
hipError_t launch_apply_bf16(const void* logits, const void* p, const int32_t* k, const void* min_p, void* out,
                          int64_t B, int64_t V, RowStrides ld, int policy, hipStream_t stream);

// p, k and min_p may each be NULL (min_p: no min-p stage).
inline hipError_t launch_apply(int dtype, const void* logits, const void* p, const int32_t* k, const void* min_p,
                               void* out, int64_t B, int64_t V, RowStrides ld, int policy, hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_apply_f32(logits, p, k, min_p, out, B, V, ld, policy, stream);
    case 1: return launch_apply_f16(logits, p, k, min_p, out, B, V, ld, policy, stream);
    case 2: return launch_apply_bf16(logits, p, k, min_p, out, B, V, ld, policy, stream);
    default: return hipErrorInvalidValue;
  }
}

// Filter plus sampling (aclnnTopKTopPSampleV2 "Subsequent processing"): q
// [B, ld_q] fp32 or NULL (None mode), out optional, selected [B] int32.
hipError_t launch_sample_f32(const void* logits, const void* p, const int32_t* k, const void* min_p, const float* q,
                             int64_t ld_q, float eps, void* out, int32_t* selected, int64_t B, int64_t V,
                             RowStrides ld, int policy, hipStream_t stream);
hipError_t launch_sample_f16(const void* logits, const void* p, const int32_t* k, const void* min_p, const float* q,
                             int64_t ld_q, float eps, void* out, int32_t* selected, int64_t B, int64_t V,
                             RowStrides ld, int policy, hipStream_t stream);
hipError_t launch_sample_bf16(const void* logits, const void* p, const int32_t* k, const void* min_p, const float* q,
                              int64_t ld_q, float eps, void* out, int32_t* selected, int64_t B, int64_t V,
                              RowStrides ld, int policy, hipStream_t stream);

inline hipError_t launch_sample(int dtype, const void* logits, const void* p, const int32_t* k, const void* min_p,
                                const float* q, int64_t ld_q, float eps, void* out, int32_t* selected, int64_t B,
                                int64_t V, RowStrides ld, int policy, hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_sample_f32(logits, p, k, min_p, q, ld_q, eps, out, selected, B, V, ld, policy, stream);
    case 1: return launch_sample_f16(logits, p, k, min_p, q, ld_q, eps, out, selected, B, V, ld, policy, stream);
    case 2: return launch_sample_bf16(logits, p, k, min_p, q, ld_q, eps, out, selected, B, V, ld, policy, stream);
    default: return hipErrorInvalidValue;
  }
}

// selected[b] = 0 for every row (rows of one element), as a kernel so that a
// caller may capture the call in a graph.
hipError_t launch_fill_zero_i32(int32_t* dst, int64_t n, hipStream_t stream);

hipError_t launch_with_sorted(int dtype, const void* sorted_value, const int32_t* sorted_indices, const void* p,
                              const int32_t* k, const void* min_p, const void* logits, void* out, int64_t B,
                              int64_t V, RowStrides ld, hipStream_t stream);

}  // namespace tkp
