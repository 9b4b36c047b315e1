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

}  // namespace tkp
