// Shared device helpers for the MoBA gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moba {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 <-> fp32.  bf16 -> fp32 is exact (the bf16 bits are the high half).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (gfx950 converts natively).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
// Two values in one packed conversion (a per-value cast costs a conversion,
// a shift and an or per pair).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Global -> LDS DMA, 16 bytes per lane: lane l's bytes come from
// base + 16 unit and land at dst + 16 l (base and dst wave-uniform; 16 unit
// below 4 GiB: the buffer offset arithmetic is 32-bit).  This is the buffer
// (MUBUF) form of the load with a 16-byte record stride.  The global (FLAT)
// form takes a full address per lane, but the compiler's wait bookkeeping
// counts a FLAT load to LDS as possibly touching LDS through the scalar-and-
// LDS counter too; while one is in flight it then waits for every LDS read
// outstanding (lgkmcnt(0)) before any LDS operand is used, which flattens the
// operand prefetch of the MFMA loops.
constexpr int kBufferWord3 = 0x00020000;  // 32-bit raw data format, gfx9 family
typedef __attribute__((address_space(3))) void lds_dma_t;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dma_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 16, -1, kBufferWord3);
}
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, uint32_t unit, void* dst) {
  __builtin_amdgcn_struct_ptr_buffer_load_lds(r, (lds_dma_t*)dst, 16, unit, 0, 0, 0, 0);
}
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t unit, void* dst) {
  lds_dma16(dma_rsrc(base), unit, dst);
}

// fp16 <-> fp32 (round to nearest even); the pair in one packed conversion.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t));
}
__device__ __forceinline__ float lo_f16(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xffffu));
}
__device__ __forceinline__ float hi_f16(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// V is staged in fp16 for the PV products, scaled per head by 2^-e so that
// the head's largest |v| lands in [2^14, 2^15), whatever the head's
// magnitude: small heads are scaled up, large ones down.  The largest staged
// value then stays below the fp16 limit, and every value of at least 2^-28
// times the head's largest is a normal fp16 number.  The scale is a power of
// two and fp16 carries more significand bits than bf16, so such a value
// converts exactly; smaller ones round to fp16 subnormals (their share of any
// output is below 2^-28 of the head's scale).  vmax_bits is the fp32 bit
// pattern of the head's largest |v|, and vmax < 2^x with x from its exponent
// field.  e is clamped at -126 so that 2^-e stays a finite fp32 number: a
// head of zeros, or one whose largest value is subnormal, takes the largest
// scale-up.
__device__ __forceinline__ int v_exponent(uint32_t vmax_bits) {
  const int x = (int)((vmax_bits >> 23) & 0xffu) - 126;  // vmax < 2^x
  return max(-126, x - 15);
}

// Index of the sequence that owns global block `gb` (largest s with
// cu_blocks[s] <= gb).  cu_blocks is non-decreasing with num_seqs + 1 entries.
__device__ __forceinline__ int seq_of_block(const int32_t* __restrict__ cu_blocks,
                                            int num_seqs, int gb) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu_blocks[mid] <= gb) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Largest i in [0, n) with arr[i] <= x for a non-decreasing arr (arr[0] <= x).
__device__ __forceinline__ int upper_index(const int32_t* __restrict__ arr, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (arr[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Length of sequence s clamped to the packed batch.
__device__ __forceinline__ void seq_span(const int32_t* __restrict__ cu_seqlens, int s,
                                         int total_tokens, int* start, int* len) {
  int a = cu_seqlens[s];
  int b = cu_seqlens[s + 1];
  a = min(max(a, 0), total_tokens);
  b = min(max(b, a), total_tokens);
  *start = a;
  *len = b - a;
}

// Walks a block_idx row and reports, for each entry, whether it is a
// historical selection (0 <= e < c, larger than the previous accepted entry,
// and among the first topk - 1 such entries).  Accepted historical entries
// get consecutive slots 0 .. topk - 2; the own block always uses slot
// topk - 1.  The bucketing passes and the merge apply exactly this rule.
__device__ __forceinline__ bool accept_hist(int e, int c, int last, int nh, int topk) {
  return e >= 0 && e < c && e > last && nh < topk - 1;
}
__device__ __forceinline__ int count_hist(const int32_t* __restrict__ row, int topk, int c) {
  int nh = 0, last = -1;
  auto visit = [&](int e) {
    if (accept_hist(e, c, last, nh, topk)) { ++nh; last = e; }
  };
  if ((topk & 3) == 0) {  // rows are 16-byte aligned: whole int4 loads
    for (int j = 0; j < topk; j += 4) {
      const int4 e4 = *reinterpret_cast<const int4*>(row + j);
      visit(e4.x);
      visit(e4.y);
      visit(e4.z);
      visit(e4.w);
    }
  } else {
    for (int j = 0; j < topk; ++j) visit(row[j]);
  }
  return nh;
}

// A row whose own block c is below dense_blocks and that selects every past
// block 0 .. c - 1 attends to its whole causal prefix [0, t]: the forward's
// dense-prefix pass writes it, and the bucketing, own-block and merge passes
// skip it (dense_blocks 0: no such rows).
__device__ __forceinline__ bool dense_row(const int32_t* __restrict__ row, int topk, int c,
                                          int dense_blocks) {
  return c < dense_blocks && count_hist(row, topk, c) == c;
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2): workgroup b runs on XCD b % 8.  xcd_remap(b, n) gives workgroup b the
// work item that makes every XCD process one contiguous share of [0, n), so
// neighbouring work items (which read the same K/V blocks) share an L2.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_remap(int b, int n) {
  const int x = b % kXcds, j = b / kXcds;
  return x * (n / kXcds) + min(x, n % kXcds) + j;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace moba
