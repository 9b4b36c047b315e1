// Small helper kernels of the C ABI.

#include "launch.h"

namespace tkp {

__global__ void fill_zero_i32_kernel(int32_t* __restrict__ dst, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = 0;
}

hipError_t launch_fill_zero_i32(int32_t* dst, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const unsigned blocks = static_cast<unsigned>((n + 255) / 256);
  hipLaunchKernelGGL(fill_zero_i32_kernel, dim3(blocks), dim3(256), 0, stream, dst, n);
  return hipGetLastError();
}

// Sorted survivors of rows of one element: that element, probability 1.
__global__ void survivors_single_kernel(float* __restrict__ probs, int32_t* __restrict__ indices,
                                        int32_t* __restrict__ counts, int64_t B, int64_t cap) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= B * cap) return;
  const int64_t r = i % cap;
  indices[i] = r == 0 ? 0 : -1;
  if (probs != nullptr) probs[i] = r == 0 ? 1.0f : 0.0f;
  if (r == 0) counts[i / cap] = 1;
}

hipError_t launch_survivors_single(float* probs, int32_t* indices, int32_t* counts, int64_t B, int64_t cap,
                                   hipStream_t stream) {
  const int64_t n = B * cap;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(survivors_single_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream,
                     probs, indices, counts, B, cap);
  return hipGetLastError();
}

}  // namespace tkp
