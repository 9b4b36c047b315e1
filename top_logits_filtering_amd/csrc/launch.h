// Internal launchers behind the C ABI. Each enqueues on `stream` and returns
// the HIP status of the launch. Shapes are already validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tkp {

// Blocks per launch at most: 2^21 blocks of 1024 threads keep a grid below
// 2^32 work-items. Larger batches are launched in row chunks.
constexpr int64_t kMaxLaunchBlocks = int64_t{1} << 21;

// 0: candidate plan, row in registers when it fits; 1: multi-pass plan only,
// row re-read from global memory; 2: candidate plan with the row re-read from
// global memory even when it would fit in registers.
enum PlanPolicy : int { kPlanAuto = 0, kPlanGeneral = 1, kPlanStream = 2 };

// Elements between the starts of consecutive rows of each [B, V] operand
// (each >= V; V when the operand is dense). `elementwise` selects the filter
// kernel for arbitrary strided views, which also reads the element strides:
// along a row of logits and out, and between the rows' entries of p, k and
// min_p (0 shares one entry among all rows).
struct RowStrides {
  int64_t x;   // logits
  int64_t o;   // out
  int64_t sv;  // sorted_value
  int64_t si;  // sorted_indices
  bool elementwise = false;
  int64_t xc = 1, oc = 1;          // element strides of logits and out
  int64_t pc = 1, kc = 1, mc = 1;  // entry strides of p, k and min_p
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

// What follows the filter (aclnnTopKTopPSampleV2 "Subsequent processing"):
// sampling into sel (q NULL: the argmax; else QSample with eps), or the
// sorted survivors into probs / indices / counts (indices not NULL).
struct SampleArgs {
  const float* q;     // [B, ld_q] fp32, or NULL
  int64_t ld_q;       // row stride of q in elements
  float eps;
  int32_t* sel;       // [B] selected original index, or NULL
  float* probs;       // [B, cap] survivors' probabilities in descending order, or NULL (sorted-survivors output)
  int32_t* indices;   // [B, cap] their original indices
  int32_t* counts;    // [B] survivors per row
  int64_t cap;
};

// Filter plus the stage above; out (the filtered logits) may be NULL.
hipError_t launch_sample_f32(const void* logits, const void* p, const int32_t* k, const void* min_p, void* out,
                             int64_t B, int64_t V, RowStrides ld, int policy, hipStream_t stream,
                             const SampleArgs& sa);
hipError_t launch_sample_f16(const void* logits, const void* p, const int32_t* k, const void* min_p, void* out,
                             int64_t B, int64_t V, RowStrides ld, int policy, hipStream_t stream,
                             const SampleArgs& sa);
hipError_t launch_sample_bf16(const void* logits, const void* p, const int32_t* k, const void* min_p, void* out,
                              int64_t B, int64_t V, RowStrides ld, int policy, hipStream_t stream,
                              const SampleArgs& sa);

inline hipError_t launch_sample(int dtype, const void* logits, const void* p, const int32_t* k, const void* min_p,
                                void* out, int64_t B, int64_t V, RowStrides ld, int policy, hipStream_t stream,
                                const SampleArgs& sa) {
  switch (dtype) {
    case 0: return launch_sample_f32(logits, p, k, min_p, out, B, V, ld, policy, stream, sa);
    case 1: return launch_sample_f16(logits, p, k, min_p, out, B, V, ld, policy, stream, sa);
    case 2: return launch_sample_bf16(logits, p, k, min_p, out, B, V, ld, policy, stream, sa);
    default: return hipErrorInvalidValue;
  }
}

// selected[b] = 0 for every row (rows of one element), as a kernel so that a
// caller may capture the call in a graph.
hipError_t launch_fill_zero_i32(int32_t* dst, int64_t n, hipStream_t stream);

// out[b * dst_stride] = src[b * src_stride] for b < B, elements of es bytes:
// strided views with rows of one element (any stride, 0 included).
hipError_t launch_copy_column(const void* src, int64_t src_stride, void* dst, int64_t dst_stride, int64_t B, int es,
                              hipStream_t stream);

// Sorted survivors of rows of one element.
hipError_t launch_survivors_single(float* probs, int32_t* indices, int32_t* counts, int64_t B, int64_t cap,
                                   hipStream_t stream);

hipError_t launch_with_sorted(int dtype, const void* sorted_value, const int32_t* sorted_indices, const void* p,
                              const int32_t* k, const void* min_p, const void* logits, void* out, int64_t B,
                              int64_t V, RowStrides ld, hipStream_t stream);

}  // namespace tkp
