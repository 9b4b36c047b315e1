// Internal launchers behind the C ABI. Each enqueues on `stream` and returns
// the HIP status of the launch. Shapes are already validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tkp {

enum PlanPolicy : int { kPlanAuto = 0, kPlanGeneral = 1, kPlanRegisters = 2 };

hipError_t launch_apply(int dtype, const void* logits, const void* p, const int32_t* k, void* out, int64_t B,
                        int64_t V, int policy, hipStream_t stream);

hipError_t launch_with_sorted(int dtype, const void* sorted_value, const int32_t* sorted_indices, const void* p,
                              const int32_t* k, const void* logits, void* out, int64_t B, int64_t V,
                              hipStream_t stream);

}  // namespace tkp
