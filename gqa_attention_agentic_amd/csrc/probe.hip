// Achievable-peak probes for gfx950 (measurement only; no part of the
// attention path uses them). They give the two ceilings the attention
// kernels are measured against on the machine at hand, next to the
// published peaks:
//  * mfma_chains: every wave keeps four independent accumulator chains of
//    v_mfma_f32_32x32x16_bf16 busy (the instruction the attention kernels'
//    products use); FLOPs = waves x iterations x 4 x 32 x 32 x 16 x 2.
//  * stream_read: a grid-stride read of a buffer with 16-byte loads, folded
//    into one word per thread so the loads cannot be dropped; bytes = the
//    buffer's size.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace gqa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(256) mfma_chains(float* out, int iters, float seed) {
  bf16x8_t a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(seed * (float)(threadIdx.x + e));
    b[e] = (__bf16)(seed * (float)(threadIdx.x - e));
  }
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ void __launch_bounds__(256) stream_read(const uint4* __restrict__ src, int64_t n16, uint32_t* out) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 x0 = src[i], x1 = src[i + stride], x2 = src[i + 2 * stride], x3 = src[i + 3 * stride];
    acc ^= x0.x ^ x0.y ^ x0.z ^ x0.w ^ x1.x ^ x1.y ^ x1.z ^ x1.w;
    acc ^= x2.x ^ x2.y ^ x2.z ^ x2.w ^ x3.x ^ x3.y ^ x3.z ^ x3.w;
  }
  for (; i < n16; i += stride) {
    const uint4 x = src[i];
    acc ^= x.x ^ x.y ^ x.z ^ x.w;
  }
  out[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

}  // namespace

hipError_t launch_probe_mfma(float* out, int blocks, int iters, hipStream_t st, hipEvent_t e0, hipEvent_t e1) {
  hipExtLaunchKernelGGL(mfma_chains, dim3(blocks), dim3(256), 0, st, e0, e1, 0, out, iters, 1e-3f);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, int64_t bytes, uint32_t* out, int blocks, hipStream_t st, hipEvent_t e0,
                             hipEvent_t e1) {
  hipExtLaunchKernelGGL(stream_read, dim3(blocks), dim3(256), 0, st, e0, e1, 0, (const uint4*)src, bytes / 16, out);
  return hipGetLastError();
}

}  // namespace gqa
