// Measurement support: sustained bf16 MFMA rate probes (not part of the
// attention).  Every wave runs four independent chains of
// v_mfma_f32_32x32x16_bf16, so the matrix pipe never waits on a dependency.
// Three operand kinds:
//   kFixed     one low-entropy operand pair held in registers for the whole
//              run (the products barely toggle the multipliers)
//   kRandom    random bf16 operands cycling through eight register sets, so
//              consecutive products see unrelated data, as attention does
//   kRandomLds random register A operands and a random B operand read from
//              LDS for every product (1 KiB per wave per MFMA, conflict
//              free), as the attention kernels feed K and V^T
// The rate each reaches is the throughput the chip sustains at the clock it
// holds under that load, to set next to the published peak.
#include "common.h"
#include "launch.h"

namespace moba {

namespace {

constexpr int kFixed = 0, kRandom = 1, kRandomLds = 2;
constexpr int kSets = 8;

// 32-bit integer hash (the "lowbias32" mixer: xor-shift / multiply rounds)
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352du;
  x ^= x >> 15; x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// uniform in [-1, 1), rounded to bf16
__device__ __forceinline__ __bf16 rand_bf16(uint32_t key) {
  return (__bf16)((float)(int32_t)mix32(key) * 0x1p-31f);
}

__device__ __forceinline__ bf16x8 rand_frag(uint32_t key) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = rand_bf16(key * 8u + (uint32_t)i);
  return r;
}

}  // namespace

template <int KIND>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void mfma_rate_kernel(int iterations, float* __restrict__ sink) {
  const int t = threadIdx.x;
  const uint32_t g = blockIdx.x * 256u + (uint32_t)t;
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  if constexpr (KIND == kFixed) {
    bf16x8 x, y;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] = (__bf16)(1e-3f * (float)((t + i) & 15));
      y[i] = (__bf16)(1e-3f * (float)((t * 3 + i) & 15));
    }
    for (int it = 0; it < iterations; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(y, x, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, x, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(y, y, c3, 0, 0, 0);
    }
  } else if constexpr (KIND == kRandom) {
    bf16x8 xs[kSets], ys[kSets];
#pragma unroll
    for (int s = 0; s < kSets; ++s) {
      xs[s] = rand_frag(g * (2 * kSets) + 2 * s);
      ys[s] = rand_frag(g * (2 * kSets) + 2 * s + 1);
    }
    // iterations counts groups of four products per wave, as for kFixed
    const int rounds = iterations / kSets;
    for (int it = 0; it < rounds; ++it) {
#pragma unroll
      for (int j = 0; j < kSets; ++j) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xs[j], ys[(j + 1) % kSets], c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xs[(j + 3) % kSets], ys[(j + 5) % kSets], c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xs[(j + 5) % kSets], ys[j], c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xs[(j + 6) % kSets], ys[(j + 2) % kSets], c3, 0, 0, 0);
      }
    }
  } else {
    // 8 KiB of random bf16 per wave: eight 1-KiB B fragments, lane l's 16
    // bytes of fragment f at byte (w * 8 + f) * 1024 + 16 l
    __shared__ __attribute__((aligned(16))) bf16x8 lds[4 * kSets * 64];
    const int w = t >> 6, lane = t & 63;
#pragma unroll
    for (int f = 0; f < kSets; ++f)
      lds[(w * kSets + f) * 64 + lane] = rand_frag(g * (3 * kSets) + 2 * kSets + f);
    bf16x8 xs[kSets];
#pragma unroll
    for (int s = 0; s < kSets; ++s) xs[s] = rand_frag(g * (3 * kSets) + s);
    __syncthreads();
    const int base = (w * kSets) * 64 + lane;
    // eight B fragments are read while the previous eight products run
    // (software pipelined through two register sets, as the attention
    // prefetches its operands)
    bf16x8 p0[kSets], p1[kSets];
#pragma unroll
    for (int f = 0; f < kSets; ++f) p0[f] = lds[base + f * 64];
    auto products = [&](const bf16x8* bs) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xs[4 * j], bs[4 * j], c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xs[4 * j + 1], bs[4 * j + 1], c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xs[4 * j + 2], bs[4 * j + 2], c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xs[4 * j + 3], bs[4 * j + 3], c3, 0, 0, 0);
      }
    };
    const int rounds = iterations / 4;  // 4 groups of 4 products per round
    for (int it = 0; it < rounds; ++it) {
      // an opaque copy of the offset keeps the reads in the loop
      int b = base;
      asm volatile("" : "+v"(b));
#pragma unroll
      for (int f = 0; f < kSets; ++f) p1[f] = lds[b + f * 64];
      __builtin_amdgcn_sched_barrier(0);  // keeps the reads ahead of the products
      products(p0);
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" : "+v"(b));
#pragma unroll
      for (int f = 0; f < kSets; ++f) p0[f] = lds[b + f * 64];
      __builtin_amdgcn_sched_barrier(0);
      products(p1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  sink[(size_t)blockIdx.x * blockDim.x + t] = s;
}

hipError_t launch_mfma_rate(int workgroups, int iterations, int operands, float* sink,
                            hipStream_t st) {
  switch (operands) {
    case kFixed:
      hipLaunchKernelGGL(mfma_rate_kernel<kFixed>, dim3(workgroups), dim3(256), 0, st,
                         iterations, sink);
      break;
    case kRandom:
      hipLaunchKernelGGL(mfma_rate_kernel<kRandom>, dim3(workgroups), dim3(256), 0, st,
                         iterations, sink);
      break;
    default:
      hipLaunchKernelGGL(mfma_rate_kernel<kRandomLds>, dim3(workgroups), dim3(256), 0, st,
                         iterations, sink);
      break;
  }
  return hipGetLastError();
}

}  // namespace moba
