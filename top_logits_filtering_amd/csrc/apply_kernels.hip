// Row filter on raw logits: the aclnn entry of the ApplyTopKTopPWithSorted
// guide (§5, §6.1), which sorts each row and then filters it. No sort is
// materialised here: each row's threshold pair (K, I) comes from radix
// selection (row_select.h) and one pass writes value-or-(-inf) in the
// original order.
//
// One 1024-thread block owns one row, so rows never exchange data and no
// global scratch is needed.
//
// Plan "general": every selection pass re-reads the row from global memory
// (the second and later reads normally hit L2 or the Infinity Cache). It
// handles any row length up to 2^20.

#include "launch.h"
#include "row_select.h"

namespace tkp {

template <class DT>
struct GlobalRowSrc {
  using raw_t = typename DT::raw_t;
  const raw_t* __restrict__ row;
  int V;
  template <class F>
  __device__ inline void for_each(F&& f) const {
    for (int i = threadIdx.x; i < V; i += kThreads) f(row[i], i);
  }
};

template <class DT>
__global__ __launch_bounds__(kThreads) void apply_general_kernel(const typename DT::raw_t* __restrict__ logits,
                                                                 const typename DT::raw_t* __restrict__ p,
                                                                 const int32_t* __restrict__ k,
                                                                 typename DT::raw_t* __restrict__ out, int V) {
  using raw_t = typename DT::raw_t;
  __shared__ RowSmem sm;
  const int b = blockIdx.x;
  const RowParams rp = decode_row_params<DT>(p, k, b, V);
  const GlobalRowSrc<DT> src{logits + static_cast<size_t>(b) * V, V};
  uint32_t K, I;
  solve_row<DT>(src, rp, sm, K, I);
  raw_t* __restrict__ o = out + static_cast<size_t>(b) * V;
  for (int i = threadIdx.x; i < V; i += kThreads) {
    const raw_t r = src.row[i];
    const uint32_t key = DT::key(r);
    o[i] = (key > K || (key == K && static_cast<uint32_t>(i) >= I)) ? r : DT::kNegInf;
  }
}

template <class DT>
static hipError_t launch_apply_t(const void* logits, const void* p, const int32_t* k, void* out, int64_t B,
                                 int64_t V, int policy, hipStream_t stream) {
  using raw_t = typename DT::raw_t;
  (void)policy;
  hipLaunchKernelGGL(apply_general_kernel<DT>, dim3(static_cast<unsigned>(B)), dim3(kThreads), 0, stream,
                     static_cast<const raw_t*>(logits), static_cast<const raw_t*>(p), k, static_cast<raw_t*>(out),
                     static_cast<int>(V));
  return hipGetLastError();
}

hipError_t launch_apply(int dtype, const void* logits, const void* p, const int32_t* k, void* out, int64_t B,
                        int64_t V, int policy, hipStream_t stream) {
  switch (dtype) {
    case 0: return launch_apply_t<F32T>(logits, p, k, out, B, V, policy, stream);
    case 1: return launch_apply_t<F16T>(logits, p, k, out, B, V, policy, stream);
    case 2: return launch_apply_t<BF16T>(logits, p, k, out, B, V, policy, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tkp
