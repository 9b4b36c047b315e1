// apply_top_k_top_p kernels instantiated for f16 (one file per dtype so
// the three builds run in parallel).

#include "apply_kernels.h"

namespace tkp {

hipError_t launch_apply_f16(const void* logits, const void* p, const int32_t* k, const void* min_p, void* out,
                          int64_t B, int64_t V, RowStrides ld, int policy, hipStream_t stream) {
  return launch_apply_t<F16T>(logits, p, k, min_p, out, B, V, ld, policy, stream);
}

hipError_t launch_sample_f16(const void* logits, const void* p, const int32_t* k, const void* min_p, void* out,
                          int64_t B, int64_t V, RowStrides ld, int policy, hipStream_t stream, const SampleArgs& sa) {
  return launch_apply_t<F16T, true>(logits, p, k, min_p, out, B, V, ld, policy, stream, sa);
}

}  // namespace tkp
