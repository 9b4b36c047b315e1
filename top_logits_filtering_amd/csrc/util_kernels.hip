// Small helper kernels of the C ABI.

#include "launch.h"

namespace tkp {

// Element kernels stride over any count with a grid of at most this many
// 256-thread blocks.
constexpr int64_t kElemBlocks = 8192;

unsigned elem_grid(int64_t n) {
  const int64_t blocks = (n + 255) / 256;
  return static_cast<unsigned>(blocks < kElemBlocks ? blocks : kElemBlocks);
}

__global__ void fill_zero_i32_kernel(int32_t* __restrict__ dst, int64_t n) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = 0;
}

hipError_t launch_fill_zero_i32(int32_t* dst, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_i32_kernel, dim3(elem_grid(n)), dim3(256), 0, stream, dst, n);
  return hipGetLastError();
}

// Sorted survivors of rows of one element: that element, probability 1.
__global__ void survivors_single_kernel(float* __restrict__ probs, int32_t* __restrict__ indices,
                                        int32_t* __restrict__ counts, int64_t B, int64_t cap) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < B * cap; i += stride) {
    const int64_t r = i % cap;
    indices[i] = r == 0 ? 0 : -1;
    if (probs != nullptr) probs[i] = r == 0 ? 1.0f : 0.0f;
    if (r == 0) counts[i / cap] = 1;
  }
}

hipError_t launch_survivors_single(float* probs, int32_t* indices, int32_t* counts, int64_t B, int64_t cap,
                                   hipStream_t stream) {
  const int64_t n = B * cap;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(survivors_single_kernel, dim3(elem_grid(n)), dim3(256), 0, stream, probs, indices, counts, B,
                     cap);
  return hipGetLastError();
}

// Rows of one element of a strided view: out[b * dst_stride] = src[b * src_stride],
// elements of es bytes (2 or 4); a source stride of 0 repeats one element.
__global__ void copy_column_kernel(const uint8_t* __restrict__ src, int64_t src_stride, uint8_t* __restrict__ dst,
                                   int64_t dst_stride, int64_t B, int es) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; b < B; b += stride) {
    const uint8_t* s = src + b * src_stride * es;
    uint8_t* d = dst + b * dst_stride * es;
    if (es == 4)
      *reinterpret_cast<uint32_t*>(d) = *reinterpret_cast<const uint32_t*>(s);
    else
      *reinterpret_cast<uint16_t*>(d) = *reinterpret_cast<const uint16_t*>(s);
  }
}

hipError_t launch_copy_column(const void* src, int64_t src_stride, void* dst, int64_t dst_stride, int64_t B, int es,
                              hipStream_t stream) {
  if (B <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_column_kernel, dim3(elem_grid(B)), dim3(256), 0, stream, static_cast<const uint8_t*>(src),
                     src_stride, static_cast<uint8_t*>(dst), dst_stride, B, es);
  return hipGetLastError();
}

}  // namespace tkp
