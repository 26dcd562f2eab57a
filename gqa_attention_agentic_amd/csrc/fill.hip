// Zero fill of the workspace's arrival counters. A kernel rather than
// hipMemsetAsync, so that a forward captured into a HIP graph holds only
// kernel and copy nodes.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kernels.h"

namespace gqa {
namespace {

__global__ void __launch_bounds__(256) zero_i32(int32_t* __restrict__ p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0;
}

}  // namespace

hipError_t launch_zero_i32(int32_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 1024);
  hipLaunchKernelGGL(zero_i32, dim3((unsigned)blocks), dim3(256), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace gqa
