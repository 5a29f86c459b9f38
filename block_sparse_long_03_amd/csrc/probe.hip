// Measurement support: a sustained bf16 MFMA rate probe (not part of the
// attention).  Every wave runs four independent chains of
// v_mfma_f32_32x32x16_bf16 on register operands, so the matrix pipe never
// waits on memory or on a dependency; the rate it reaches is the chip's
// sustainable dense bf16 MFMA throughput at the clock it holds under that
// load, to set next to the published peak.
#include "common.h"
#include "launch.h"

namespace moba {

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void mfma_rate_kernel(int iterations, float* __restrict__ sink) {
  const int t = threadIdx.x;
  bf16x8 x, y;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = (__bf16)(1e-3f * (float)((t + i) & 15));
    y[i] = (__bf16)(1e-3f * (float)((t * 3 + i) & 15));
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iterations; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(y, x, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, x, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(y, y, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  sink[(size_t)blockIdx.x * blockDim.x + t] = s;
}

hipError_t launch_mfma_rate(int workgroups, int iterations, float* sink, hipStream_t st) {
  hipLaunchKernelGGL(mfma_rate_kernel, dim3(workgroups), dim3(256), 0, st, iterations, sink);
  return hipGetLastError();
}

}  // namespace moba
