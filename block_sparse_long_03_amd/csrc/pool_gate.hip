// Block mean-pool of the keys and the fused gate + causal top-k selection.
//
// Pool: "MoBA: Learned Block Sparsity for Long-Context Attention", section
// "The Change" (mean_pool(K[I_i]) as the block's representative key).
// Gate: same section (s_i = <q, mean_pool(K[I_i])>, hard top-k, future blocks
// masked out of routing, own block always selected and counted in k).
#include "common.h"
#include "launch.h"

namespace moba {

// ---------------------------------------------------------------------------
// pool: kbar[gb, :] = (sum over the block's tokens of K[t, :]) / count
// One workgroup covers one block and 64 consecutive elements of the H*d row:
// 8 column threads x 8 elements, 32 token lanes each summing every 32nd
// token in fp32, then a fixed-order tree over the 32 lanes.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void load8(const T* p, float* v);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float* v) {
  u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[2 * i] = lo_bf16(w[i]); v[2 * i + 1] = hi_bf16(w[i]); }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* v) {
  f32x4 a = *reinterpret_cast<const f32x4*>(p);
  f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
}

// upper half of an fp32 pattern: x truncated to bf16 (exact as a float)
__device__ __forceinline__ float bf16_trunc(float x) {
  return __uint_as_float(__float_as_uint(x) & 0xffff0000u);
}

template <typename T>
__global__ __launch_bounds__(256) void pool_keys_kernel(
    const T* __restrict__ k, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ cu_blocks, int num_seqs, int total_tokens, int hd, int D,
    int block_size, float* __restrict__ kbar, uint16_t* __restrict__ kbar3) {
  __shared__ float red[32][65];
  const int gb = blockIdx.x;
  const int col0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 7;
  const int ty = threadIdx.x >> 3;
  const int s = seq_of_block(cu_blocks, num_seqs, gb);
  int start, len;
  seq_span(cu_seqlens, s, total_tokens, &start, &len);
  const int local = (gb - cu_blocks[s]) * block_size;
  const int cnt = min(block_size, len - local);

  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  if (cnt > 0) {
    const T* base = k + (size_t)(start + local) * hd + col0 + tx * 8;
    int j = ty;
    for (; j + 96 < cnt; j += 128) {
      float v0[8], v1[8], v2[8], v3[8];
      load8<T>(base + (size_t)j * hd, v0);
      load8<T>(base + (size_t)(j + 32) * hd, v1);
      load8<T>(base + (size_t)(j + 64) * hd, v2);
      load8<T>(base + (size_t)(j + 96) * hd, v3);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v0[i];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v1[i];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v2[i];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v3[i];
    }
    for (; j < cnt; j += 32) {
      float v0[8];
      load8<T>(base + (size_t)j * hd, v0);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v0[i];
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) red[ty][tx * 8 + i] = acc[i];
  __syncthreads();
  for (int stride = 16; stride >= 1; stride >>= 1) {
    if (ty < stride) {
#pragma unroll
      for (int i = 0; i < 8; ++i) red[ty][tx * 8 + i] += red[ty + stride][tx * 8 + i];
    }
    __syncthreads();
  }
  if (ty == 0) {
    float* dst = kbar + (size_t)gb * hd + col0 + tx * 8;
    const float inv_cnt = (float)max(cnt, 1);
    float m[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      m[i] = cnt > 0 ? red[0][tx * 8 + i] / inv_cnt : 0.f;
      dst[i] = m[i];
    }
    if (kbar3) {
      // m = hi + mid + lo exactly: hi and mid are 8-bit truncations, and the
      // rest has at most 8 significant bits, so its bf16 rounding is exact.
      // Layout [head][term][d / 16][block][16]: the 16-element k-step
      // fragments of consecutive blocks are contiguous.
      const int h = (col0 + tx * 8) / D, e0 = (col0 + tx * 8) - h * D;
      const size_t nb = gridDim.x;
      const size_t plane = (size_t)(D / 16) * nb * 16;  // one term of one head
      uint16_t* d3 = kbar3 + (size_t)h * 3 * plane + ((size_t)(e0 >> 4) * nb + gb) * 16 + (e0 & 15);
      u32x4 whi, wmid, wlo;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float h0 = bf16_trunc(m[2 * i]), h1 = bf16_trunc(m[2 * i + 1]);
        const float r0 = m[2 * i] - h0, r1 = m[2 * i + 1] - h1;
        const float m0 = bf16_trunc(r0), m1 = bf16_trunc(r1);
        whi[i] = (__float_as_uint(h0) >> 16) | (__float_as_uint(h1) & 0xffff0000u);
        wmid[i] = (__float_as_uint(m0) >> 16) | (__float_as_uint(m1) & 0xffff0000u);
        wlo[i] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(r0 - m0)) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)(r1 - m1)) << 16);
      }
      *reinterpret_cast<u32x4*>(d3) = whi;
      *reinterpret_cast<u32x4*>(d3 + plane) = wmid;
      *reinterpret_cast<u32x4*>(d3 + 2 * plane) = wlo;
    }
  }
}

// min/max pool: the elementwise max and min of the block's keys (exact: no
// rounding), stored group-major.  The [kmax, kmin] row of (block gb, head h)
// has 2 D values in 2 D / 4 groups of 4 (groups 0 .. D / 4 - 1 the max,
// D / 4 .. D / 2 - 1 the min), and group g of every block of head h is one
// run: kmm[((h * (D / 2) + g) * NB + gb) * 4 + i] = row value 4 g + i.  A
// gate wave's 32 blocks then read one group as 32 consecutive 16-byte
// records (512 bytes) instead of 32 separate lines.
template <typename T>
__global__ __launch_bounds__(256) void pool_minmax_kernel(
    const T* __restrict__ k, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ cu_blocks, int num_seqs, int total_tokens, int total_blocks,
    int hd, int D, int block_size, float* __restrict__ kmm) {
  __shared__ float rmax[32][65];
  __shared__ float rmin[32][65];
  const int gb = blockIdx.x;
  const int col0 = blockIdx.y * 64;
  const int tx = threadIdx.x & 7;
  const int ty = threadIdx.x >> 3;
  const int s = seq_of_block(cu_blocks, num_seqs, gb);
  int start, len;
  seq_span(cu_seqlens, s, total_tokens, &start, &len);
  const int local = (gb - cu_blocks[s]) * block_size;
  const int cnt = min(block_size, len - local);

  float mx[8], mn[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { mx[i] = -INFINITY; mn[i] = INFINITY; }
  if (cnt > 0) {
    const T* base = k + (size_t)(start + local) * hd + col0 + tx * 8;
    int j = ty;
    for (; j + 32 < cnt; j += 64) {
      float v0[8], v1[8];
      load8<T>(base + (size_t)j * hd, v0);
      load8<T>(base + (size_t)(j + 32) * hd, v1);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        mx[i] = fmaxf(mx[i], fmaxf(v0[i], v1[i]));
        mn[i] = fminf(mn[i], fminf(v0[i], v1[i]));
      }
    }
    for (; j < cnt; j += 32) {
      float v0[8];
      load8<T>(base + (size_t)j * hd, v0);
#pragma unroll
      for (int i = 0; i < 8; ++i) { mx[i] = fmaxf(mx[i], v0[i]); mn[i] = fminf(mn[i], v0[i]); }
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) { rmax[ty][tx * 8 + i] = mx[i]; rmin[ty][tx * 8 + i] = mn[i]; }
  __syncthreads();
  for (int stride = 16; stride >= 1; stride >>= 1) {
    if (ty < stride) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        rmax[ty][tx * 8 + i] = fmaxf(rmax[ty][tx * 8 + i], rmax[ty + stride][tx * 8 + i]);
        rmin[ty][tx * 8 + i] = fminf(rmin[ty][tx * 8 + i], rmin[ty + stride][tx * 8 + i]);
      }
    }
    __syncthreads();
  }
  if (ty == 0) {
    // column col0 + 8 tx + i of the [H * D] row is (head, dim) = divmod(col, D);
    // dims e .. e + 7 are the groups e / 4 and e / 4 + 1 of the max half and
    // D / 4 + e / 4, + 1 of the min half
    const int col = col0 + tx * 8;
    const int h = col / D, e = col - h * D;
    const size_t nbk = (size_t)total_blocks;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int gi = 0; gi < 2; ++gi) {
        f32x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = half == 0 ? rmax[0][tx * 8 + 4 * gi + i] : rmin[0][tx * 8 + 4 * gi + i];
          v[i] = cnt > 0 ? x : 0.f;
        }
        const int grp = half * (D / 4) + e / 4 + gi;
        *reinterpret_cast<f32x4*>(kmm + (((size_t)h * (D / 2) + grp) * nbk + gb) * 4) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// gate + top-k
// ---------------------------------------------------------------------------

// Order-preserving map of a finite fp32 score to uint32 (-0 folded onto +0 so
// that equal scores compare equal and ties fall to the block index).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

constexpr int kGateRows = 32;    // query tokens per workgroup (they share one own block c)
constexpr int kGateSpan = 256;   // past blocks per selection pass (4 per lane)
// Scores of block j of a span sit at column gate_col(j) of their LDS row: 4
// columns of padding after every 32, so that 16-byte reads of 8 lanes at
// block offsets 16 or 32 apart fall into distinct banks.
constexpr int kGateStride = kGateSpan + kGateSpan / 8 + 4;  // 292: 16-byte aligned rows
__device__ __forceinline__ int gate_col(int j) { return j + 4 * (j >> 5); }
constexpr int kGateFastK = 16;   // k - 1 up to this: threshold from sorted per-lane lists
constexpr int kGateChunk = 128;  // past blocks per MFMA scoring step (one 32 x 32 tile per wave)
constexpr int kGateChunkValu = 64;  // past blocks per fp32 scoring step
constexpr int kGateWaves = 4;
constexpr int kGateRowsPerWave = kGateRows / kGateWaves;
// the single-span kernel: 64 query tokens and 8 waves per workgroup; wave w
// scores block tile w for all 64 tokens
constexpr int kSpanWaves = 8;
constexpr int kSpanRows = kSpanWaves * kGateRowsPerWave;

// exact split of an fp32 value into three bf16 parts: x = hi + mid + lo
__device__ __forceinline__ void split3(float x, __bf16& hi, __bf16& mid, __bf16& lo) {
  const float h = __uint_as_float(__float_as_uint(x) & 0xffff0000u);
  const float r1 = x - h;
  const float m = __uint_as_float(__float_as_uint(r1) & 0xffff0000u);
  hi = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(h) >> 16));
  mid = __builtin_bit_cast(__bf16, (uint16_t)(__float_as_uint(m) >> 16));
  lo = (__bf16)(r1 - m);  // at most 8 significant bits remain: exact
}

// Scores of a chunk of up to 128 past blocks for the 32 query rows, written
// to ss[row][col0 + j].  bf16 queries: s = q . kbar with kbar split exactly
// into three bf16 parts and the three products summed by
// v_mfma_f32_32x32x16_bf16 (products exact, fp32 accumulation); each of the
// 4 waves owns one 32 x 32 tile (block tile w).
// bf16 fragment with every negative element (sign bit set) zeroed (NEG false)
// or every non-negative one zeroed (NEG true): q+ and q- exactly
template <bool NEG>
__device__ __forceinline__ bf16x8 sign_part(const bf16x8& x) {
  u32x4 w = __builtin_bit_cast(u32x4, x);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t m = ((w[i] >> 15) & 0x00010001u) * 0xffffu;  // 0xffff where negative
    w[i] &= NEG ? m : ~m;
  }
  return __builtin_bit_cast(bf16x8, w);
}

// QUEST: kbar rows are [kmax (D), kmin (D)] and the score is
// q+ . kmax + q- . kmin = sum_e max(q_e kmin_e, q_e kmax_e)
template <int D, bool QUEST>
__device__ __forceinline__ void gate_scores_mfma(const bf16x8 (&qfrag)[D / 16],
                                                 const float* __restrict__ kbar, int H, int h,
                                                 int gblk0, int nb, int total_blocks,
                                                 float (*ss)[kGateStride], int col0, int w,
                                                 int lane) {
  constexpr int KD = QUEST ? 2 * D : D;  // length of a kbar row
  const int l32 = lane & 31, hf = lane >> 5;
  const int bt = w & 3, tt = w >> 2;
  const int j = 32 * bt + l32;  // block of this lane's A rows
  const bool ok = j < nb && gblk0 + j < total_blocks;
  // lanes past the chunk read block gblk0 (always valid) and zero it, so the
  // loads carry no branch and can all be in flight together
  const int blk = ok ? gblk0 + j : gblk0;
  // mean keys: [NB, H, D] rows; min/max: the group-major layout of
  // pool_minmax_kernel (groups 4 ks + 2 hf and + 1 hold dims 16 ks + 8 hf .. + 7)
  const float* kp = QUEST ? kbar + (((size_t)h * (KD / 4) + 2 * hf) * total_blocks + blk) * 4
                          : kbar + ((size_t)blk * H + h) * KD + 8 * hf;
  const size_t sa = QUEST ? (size_t)total_blocks * 16 : 16;  // floats per k-step
  const size_t sb = QUEST ? (size_t)total_blocks * 4 : 4;    // second half of a k-step
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  constexpr int KH = D / 32;  // k-steps per group (loads of a group in flight together)
#pragma unroll
  for (int half = 0; half < KD / (16 * KH); ++half) {
  f32x4 xa[KH], xb[KH];
#pragma unroll
  for (int kk = 0; kk < KH; ++kk) {
    xa[kk] = *reinterpret_cast<const f32x4*>(kp + sa * (half * KH + kk));
    xb[kk] = *reinterpret_cast<const f32x4*>(kp + sa * (half * KH + kk) + sb);
  }
#pragma unroll
  for (int kk = 0; kk < KH; ++kk) {
    const int ks = half * KH + kk;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    const f32x4 x0 = ok ? xa[kk] : zero, x1 = ok ? xb[kk] : zero;
    bf16x8 hi, mid, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      __bf16 a, b, cc;
      split3(e < 4 ? x0[e] : x1[e - 4], a, b, cc);
      hi[e] = a;
      mid[e] = b;
      lo[e] = cc;
    }
    bf16x8 qb;
    if constexpr (QUEST)
      qb = ks < D / 16 ? sign_part<false>(qfrag[ks]) : sign_part<true>(qfrag[ks - D / 16]);
    else
      qb = qfrag[ks];
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, qb, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mid, qb, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, qb, acc, 0, 0, 0);
  }
  }
  // acc[r] = score of block 32 bt + 8 (r / 4) + 4 hf + (r % 4) for token 32 tt + (lane & 31)
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int jb = 32 * bt + 8 * (r >> 2) + 4 * hf + (r & 3);  // block in the chunk
    ss[32 * tt + l32][gate_col(col0 + jb)] = jb < nb ? acc[r] : -INFINITY;
  }
}

// Scores of a chunk of up to 128 past blocks from the pooled keys' bf16
// terms (hi, mid, lo; layout [head][term][d / 16][block][16], as
// moba_pool_keys writes them, so that one load of a wave reads the 32-byte
// fragments of 32 consecutive blocks, 1 KiB in a row):
// the three exact products summed in fp32 by v_mfma_f32_32x32x16_bf16, each
// wave w owning the 32 x 32 tile of block tile w % 4 and query tokens
// 32 (w / 4) .. + 31, written to ss[row][gate_col(col0 + j)].
template <int D>
__device__ __forceinline__ void gate_scores_planes(const bf16x8 (&qfrag)[D / 16],
                                                   const uint16_t* __restrict__ kbar3, int H,
                                                   int h, int gblk0, int nb, int total_blocks,
                                                   float (*ss)[kGateStride], int col0, int w,
                                                   int lane) {
  const int l32 = lane & 31, hf = lane >> 5;
  const int bt = w & 3;
  const int j = 32 * bt + l32;  // block of this lane's A rows
  const bool ok = j < nb && gblk0 + j < total_blocks;
  // lanes past the chunk read block gblk0 (always valid) and zero it
  const size_t plane = (size_t)(D / 16) * total_blocks * 16;
  const uint16_t* kp = kbar3 + (size_t)h * 3 * plane + (size_t)(ok ? gblk0 + j : gblk0) * 16 + 8 * hf;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  constexpr int KH = D / 32;  // k-steps per group of loads in flight together
#pragma unroll
  for (int half = 0; half < D / (16 * KH); ++half) {
    u32x4 a[3][KH];
#pragma unroll
    for (int kk = 0; kk < KH; ++kk)
#pragma unroll
      for (int pl = 0; pl < 3; ++pl)
        a[pl][kk] = *reinterpret_cast<const u32x4*>(
            kp + pl * plane + (size_t)(half * KH + kk) * total_blocks * 16);
#pragma unroll
    for (int kk = 0; kk < KH; ++kk) {
      const bf16x8 qb = qfrag[half * KH + kk];
#pragma unroll
      for (int pl = 0; pl < 3; ++pl) {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, ok ? a[pl][kk] : zero), qb, acc, 0, 0, 0);
      }
    }
  }
  // acc[r] = score of block 32 bt + 8 (r / 4) + 4 hf + (r % 4) for token lane & 31
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int jb = 32 * bt + 8 * (r >> 2) + 4 * hf + (r & 3);  // block in the chunk
    ss[32 * (w >> 2) + l32][gate_col(col0 + jb)] = jb < nb ? acc[r] : -INFINITY;
  }
}

// The single-span kernel's scores (at most 256 past blocks, so at most one
// 32-block tile per wave): wave w owns blocks 32 w .. 32 w + 31 for all 64
// query tokens of the workgroup, with one accumulator per 32 tokens, so each
// fragment of the pooled-key terms is fetched once per workgroup and only the
// tiles below the row's span are computed.  Per k-step the wave loads the
// three term fragments and the Q fragments of both token halves and issues six
// products; each token's score is summed in the same order as in
// gate_scores_planes (k-steps, then hi, mid, lo), so the scores are the same
// bits.  Q rows past the sequence end load as zeros.
template <int D>
__device__ __forceinline__ void gate_scores_span(const uint16_t* __restrict__ q, int start, int len,
                                                 int p0, int H, int h,
                                                 const uint16_t* __restrict__ kbar3, int gblk0,
                                                 int nb, int total_blocks,
                                                 float (*ss)[kGateStride], int w, int lane) {
  const int l32 = lane & 31, hf = lane >> 5;
  const int j = 32 * w + l32;  // block of this lane's A rows
  const bool ok = j < nb && gblk0 + j < total_blocks;
  const size_t plane = (size_t)(D / 16) * total_blocks * 16;
  const uint16_t* kp = kbar3 + (size_t)h * 3 * plane + (size_t)(ok ? gblk0 + j : gblk0) * 16 + 8 * hf;
  const uint16_t* qp[2];
  bool qv[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int tok = p0 + 32 * t + l32;
    qv[t] = tok < len;
    qp[t] = q + ((size_t)(start + (qv[t] ? tok : p0)) * H + h) * D + 8 * hf;
  }
  f32x16 acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  constexpr int KH = D / 32;  // k-steps per group of loads in flight together
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int half = 0; half < D / (16 * KH); ++half) {
    u32x4 a[3][KH], b[2][KH];
#pragma unroll
    for (int kk = 0; kk < KH; ++kk) {
#pragma unroll
      for (int pl = 0; pl < 3; ++pl)
        a[pl][kk] = *reinterpret_cast<const u32x4*>(
            kp + pl * plane + (size_t)(half * KH + kk) * total_blocks * 16);
#pragma unroll
      for (int t = 0; t < 2; ++t)
        b[t][kk] = qv[t] ? *reinterpret_cast<const u32x4*>(qp[t] + 16 * (half * KH + kk)) : zero;
    }
#pragma unroll
    for (int kk = 0; kk < KH; ++kk)
#pragma unroll
      for (int pl = 0; pl < 3; ++pl)
#pragma unroll
        for (int t = 0; t < 2; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, ok ? a[pl][kk] : zero),
              __builtin_bit_cast(bf16x8, b[t][kk]), acc[t], 0, 0, 0);
  }
  // acc[t][r] = score of block 32 w + 8 (r / 4) + 4 hf + (r % 4) for token 32 t + lane & 31
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int jb = 32 * w + 8 * (r >> 2) + 4 * hf + (r & 3);
#pragma unroll
    for (int t = 0; t < 2; ++t) ss[32 * t + l32][gate_col(jb)] = jb < nb ? acc[t][r] : -INFINITY;
  }
}

// The same tile for the min/max gate: the A rows are the fp32 [kmax, kmin]
// rows of the blocks, the B columns q+ (against kmax) and q- (against kmin).
// Each fragment is split into its three exact bf16 terms as in
// gate_scores_mfma, in the same summation order; when every element of a
// wave's fragment is a bf16 value (always, for keys pooled from bf16 inputs)
// the mid and lo terms are zero and their products are skipped.
template <int D>
__device__ __forceinline__ void gate_scores_span_minmax(const uint16_t* __restrict__ q, int start,
                                                        int len, int p0, int H, int h,
                                                        const float* __restrict__ kmm, int gblk0,
                                                        int nb, int total_blocks,
                                                        float (*ss)[kGateStride], int w,
                                                        int lane) {
  constexpr int KD = 2 * D;  // length of a [kmax, kmin] row
  const int l32 = lane & 31, hf = lane >> 5;
  const int j = 32 * w + l32;
  const bool ok = j < nb && gblk0 + j < total_blocks;
  // dims 16 ks + 8 hf .. + 7 of the block's [kmax, kmin] row: groups
  // 4 ks + 2 hf and 4 ks + 2 hf + 1 (consecutive lanes read consecutive
  // 16-byte records of one group)
  const float* kp = kmm + (((size_t)h * (KD / 4) + 2 * hf) * total_blocks + (ok ? gblk0 + j : gblk0)) * 4;
  const size_t gstep = (size_t)total_blocks * 4;  // floats between groups
  const uint16_t* qp[2];
  bool qv[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int tok = p0 + 32 * t + l32;
    qv[t] = tok < len;
    qp[t] = q + ((size_t)(start + (qv[t] ? tok : p0)) * H + h) * D + 8 * hf;
  }
  f32x16 acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[t][r] = 0.f;
  constexpr int KH = D / 64;  // k-steps per group of loads in flight together
  const f32x4 fzero = {0.f, 0.f, 0.f, 0.f};
  const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int half = 0; half < KD / (16 * KH); ++half) {
    f32x4 xa[KH], xb[KH];
    u32x4 b[2][KH];
#pragma unroll
    for (int kk = 0; kk < KH; ++kk) {
      const int ks = half * KH + kk;
      xa[kk] = *reinterpret_cast<const f32x4*>(kp + 4 * ks * gstep);
      xb[kk] = *reinterpret_cast<const f32x4*>(kp + (4 * ks + 1) * gstep);
#pragma unroll
      for (int t = 0; t < 2; ++t)
        b[t][kk] = qv[t] ? *reinterpret_cast<const u32x4*>(qp[t] + 16 * (ks % (D / 16))) : zero;
    }
#pragma unroll
    for (int kk = 0; kk < KH; ++kk) {
      const int ks = half * KH + kk;
      const f32x4 x0 = ok ? xa[kk] : fzero, x1 = ok ? xb[kk] : fzero;
      bf16x8 qb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        qb[t] = ks < D / 16 ? sign_part<false>(__builtin_bit_cast(bf16x8, b[t][kk]))
                            : sign_part<true>(__builtin_bit_cast(bf16x8, b[t][kk]));
      bf16x8 hi;
      bool exact = true;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = e < 4 ? x0[e] : x1[e - 4];
        const uint32_t hb = __float_as_uint(x) & 0xffff0000u;
        exact = exact && __uint_as_float(hb) == x;
        hi[e] = __builtin_bit_cast(__bf16, (uint16_t)(hb >> 16));
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hi, qb[t], acc[t], 0, 0, 0);
      if (__ballot(!exact) != 0ull) {
        bf16x8 mid, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          __bf16 a, bb, cc;
          split3(e < 4 ? x0[e] : x1[e - 4], a, bb, cc);
          mid[e] = bb;
          lo[e] = cc;
        }
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(mid, qb[t], acc[t], 0, 0, 0);
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lo, qb[t], acc[t], 0, 0, 0);
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int jb = 32 * w + 8 * (r >> 2) + 4 * hf + (r & 3);
#pragma unroll
    for (int t = 0; t < 2; ++t) ss[32 * t + l32][gate_col(jb)] = jb < nb ? acc[t][r] : -INFINITY;
  }
}

// fp32 queries: plain fp32 FMA over d in index order (LDS tiles of q and kbar)
template <int D, int NT>
__device__ __forceinline__ void gate_scores_valu(const float (*qs)[D + 4], float (*ks)[D + 4],
                                                 const float* __restrict__ kbar, int H, int h,
                                                 int gblk0, int nb, int total_blocks,
                                                 float (*ss)[kGateStride], int col0, int tid) {
  for (int i = tid; i < kGateChunkValu * (D / 4); i += NT) {
    const int j = i / (D / 4), e4 = i % (D / 4);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (j < nb && gblk0 + j < total_blocks)
      v = *reinterpret_cast<const f32x4*>(kbar + ((size_t)(gblk0 + j) * H + h) * D + e4 * 4);
    *reinterpret_cast<f32x4*>(&ks[j][e4 * 4]) = v;
  }
  __syncthreads();
  const int ty = tid >> 4;  // rows 2ty, 2ty+1 (NT / 8 rows)
  const int tx = tid & 15;  // blocks tx + 16 jj
  float acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;
#pragma unroll 4
  for (int e = 0; e < D; e += 4) {
    const f32x4 qa = *reinterpret_cast<const f32x4*>(&qs[2 * ty][e]);
    const f32x4 qb = *reinterpret_cast<const f32x4*>(&qs[2 * ty + 1][e]);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const f32x4 kv = *reinterpret_cast<const f32x4*>(&ks[tx + 16 * jj][e]);
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc[0][jj] = fmaf(qa[u], kv[u], acc[0][jj]);
        acc[1][jj] = fmaf(qb[u], kv[u], acc[1][jj]);
      }
    }
  }
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const bool okj = tx + 16 * jj < nb;  // columns past the chunk's blocks: -inf
    ss[2 * ty][gate_col(col0 + tx + 16 * jj)] = okj ? acc[0][jj] : -INFINITY;
    ss[2 * ty + 1][gate_col(col0 + tx + 16 * jj)] = okj ? acc[1][jj] : -INFINITY;
  }
  __syncthreads();  // ks is reused by the next chunk
}

// ---------------------------------------------------------------------------
// Candidate selection: the top k - 1 of one span of at most 256 past blocks
// for the 8 rows of a wave (8 lanes per row, lane part p = lane % 8), for
// k - 1 <= kSelMaxK.  Cheaper than ranking every key:
//  1. each lane keeps the T largest of its keys j = p, p + 8, ... (T chosen
//     with 8 T >= k - 1); the (k - 1)-th largest L of these 8 T values is a
//     lower bound of the row's (k - 1)-th largest key, with at least k - 1
//     keys >= L;
//  2. the keys >= L (the candidates: about k of them for Gaussian-like
//     scores) are marked in bitmaps over contiguous block ranges and their
//     block ids compacted into LDS in ascending order;
//  3. a bitonic sort of at most 8 CL candidates (CL per lane) gives the
//     exact (k - 1)-th largest key t, and the selection is every candidate
//     above t plus the lowest-index candidates equal to t.  When every row
//     of the wave has exactly k - 1 candidates (usual for T = 8) they are
//     the selection and the sort is skipped.
// A row with more than 8 CL candidates (ties, degenerate scores) makes
// the wave return false before writing anything; the general paths then
// handle its rows.  Keys are the fp32 scores themselves (-0 and +0 compare
// equal, as the order keys of the other paths make them); scores are finite,
// and the score columns of a span past its last block hold -inf (the
// scoring writes whole chunks), so the passes run over whole groups of 32
// blocks.  Maxima, minima and medians are v_med3_f32: the i-th largest of
// {t_0 >= .. >= t_(T-1), x} is med3(t_(i-1), t_i, x), and a compare-exchange
// is med3(a, b, -inf) (min) or med3(a, b, +inf) (max).
// ---------------------------------------------------------------------------
constexpr int kSelMaxK = 40;  // k - 1 up to this
constexpr int kSelCap = 64;   // candidate slots per row in LDS (at most 8 per lane)

__device__ __forceinline__ float med3(float a, float b, float c) {
  return __builtin_amdgcn_fmed3f(a, b, c);
}
// +-inf in a register the compiler cannot see into: med3 with a known
// infinity would be folded into fmax / fmin, which canonicalise their inputs
// with an extra instruction each
__device__ __forceinline__ float opaque(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Lane exchanges inside groups of 8 lanes as DPP moves (VALU, no LDS round
// trip): quad_perm [1,0,3,2] and [2,3,0,1] are lane ^ 1 and lane ^ 2;
// lane ^ 4 is quad_perm [3,2,1,0] (lane ^ 3) followed by row_half_mirror
// (lane 7 - i of each 8, i.e. lane ^ 7).  row_shr:d gives lane i the value
// of lane i - d of its 16-lane row (lanes below d in their group of 8 get
// another group's value, which the callers ignore).  Against ds_bpermute
// shuffles: 1M gate 9.14 -> 8.80 ms, 32K 0.260 -> 0.249 ms, same selections.
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppXor3 = 0x1B, kDppHalfMirror = 0x141;
constexpr int kDppRowShr = 0x110;
__device__ __forceinline__ float group_xor(float v, int m) {
  const int x = __float_as_int(v);
  if (m == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(x, kDppXor1, 0xF, 0xF, false));
  if (m == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(x, kDppXor2, 0xF, 0xF, false));
  const int y = __builtin_amdgcn_mov_dpp(x, kDppXor3, 0xF, 0xF, false);
  return __int_as_float(__builtin_amdgcn_mov_dpp(y, kDppHalfMirror, 0xF, 0xF, false));
}
__device__ __forceinline__ int group_shr(int x, int d) {
  if (d == 1) return __builtin_amdgcn_mov_dpp(x, kDppRowShr + 1, 0xF, 0xF, false);
  if (d == 2) return __builtin_amdgcn_mov_dpp(x, kDppRowShr + 2, 0xF, 0xF, false);
  return __builtin_amdgcn_mov_dpp(x, kDppRowShr + 4, 0xF, 0xF, false);
}

// Ascending bitonic sort of the 8 N values v[i] of lanes 8 g .. 8 g + 7 (value
// index p N + i); N a power of two.
template <int N>
__device__ __forceinline__ void group_sort_asc(float (&v)[N], int p, float pinf, float ninf) {
#pragma unroll
  for (int k = 2; k <= 8 * N; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= N) {
#pragma unroll
        for (int i = 0; i < N; ++i) {
          const float o = group_xor(v[i], j / N);
          const int g = p * N + i;
          const bool keep_min = ((g & k) == 0) == ((g & j) == 0);
          v[i] = med3(v[i], o, keep_min ? ninf : pinf);
        }
      } else {
#pragma unroll
        for (int i = 0; i < N; ++i) {
          if ((i & j) == 0) {
            const bool up = ((p * N + i) & k) == 0;
            const float a = v[i], b = v[i + j];
            v[i] = med3(a, b, up ? ninf : pinf);
            v[i + j] = med3(a, b, up ? pinf : ninf);
          }
        }
      }
    }
  }
}

// Sum of v over the 8 lanes of the group; *excl = sum over the lanes below.
__device__ __forceinline__ int group_scan(int v, int p, int* excl) {
  int inc = v;
#pragma unroll
  for (int d = 1; d < 8; d <<= 1) {
    const int u = group_shr(inc, d);
    if (p >= d) inc += u;
  }
  *excl = inc - v;
  // lane 7 of each group of 8: ds_swizzle in bit mode, source lane
  // (i & 0x18) | 7 of each 32
  return __builtin_amdgcn_ds_swizzle(inc, 0x18 | (7 << 5));
}

// Element `idx` (uniform) of the ascending order of a group sort.
template <int N>
__device__ __forceinline__ float group_pick(const float (&v)[N], int idx, int lane) {
  float e = v[0];
#pragma unroll
  for (int i = 1; i < N; ++i) e = (idx % N == i) ? v[i] : e;
  return __shfl(e, (lane & ~7) | (idx / N));
}

template <int T, int CL>
__device__ __forceinline__ bool gate_select_candidates(const float (*ss)[kGateStride],
                                                       uint8_t (*cand)[kSelCap], int w, int lane,
                                                       int nq, int nspan, int k1, int topk, int c,
                                                       int32_t* __restrict__ rows0,
                                                       int row_stride) {
  static_assert(CL == 4 || CL == 8, "4 or 8 candidates per lane");
  constexpr int kCap = 8 * CL;
  const int rr = lane >> 3, p = lane & 7;
  const int r = w * kGateRowsPerWave + rr;
  const bool rv = r < nq;
  const float* srow = ss[r];  // rows past the tile end hold defined scores (zero queries)
  const int ng = (nspan + 31) >> 5;  // groups of 32 blocks
  const float pinf = opaque(INFINITY), ninf = opaque(-INFINITY);
  // 1. the lane's T largest keys (blocks 32 g + p + 8 i at column 36 g + p + 8 i), and L
  float top[T];
#pragma unroll
  for (int i = 0; i < T; ++i) top[i] = -INFINITY;
  for (int g = 0; g < ng; ++g) {
    const float* b = srow + 36 * g + p;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x = b[8 * i];
      float nt[T];
      nt[0] = med3(top[0], x, pinf);
#pragma unroll
      for (int s = 1; s < T; ++s) nt[s] = med3(top[s - 1], top[s], x);
#pragma unroll
      for (int s = 0; s < T; ++s) top[s] = nt[s];
    }
  }
  group_sort_asc<T>(top, p, pinf, ninf);
  const float L = group_pick<T>(top, 8 * T - k1, lane);  // finite: the span has > k1 blocks
  // 2. candidate bitmaps: lane p covers blocks [p R, p R + R), bit m = block p R + m
  const int R = 4 * ng;
  uint32_t bits = 0u;
  for (int qd = 0; qd < ng; ++qd) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(srow + gate_col(p * R + 4 * qd));
#pragma unroll
    for (int e = 0; e < 4; ++e) bits |= (uint32_t)(v[e] >= L) << (4 * qd + e);
  }
  if (!rv) bits = 0u;
  int excl;
  const int total = group_scan(__popc(bits), p, &excl);
  if (__ballot(total > kCap) != 0ull) return false;
  uint8_t* crow = cand[rr];
  __builtin_amdgcn_wave_barrier();
  {
    int pos = excl;
    for (uint32_t b = bits; b != 0u; b &= b - 1u) crow[pos++] = (uint8_t)(p * R + __builtin_ctz(b));
  }
  __builtin_amdgcn_wave_barrier();
  // 3. the exact threshold among the candidates (positions CL p .. CL p + CL - 1)
  uint32_t cw[CL / 4];
  if constexpr (CL == 4) {
    cw[0] = *reinterpret_cast<const uint32_t*>(crow + 4 * p);
  } else {
    const uint2 c8 = *reinterpret_cast<const uint2*>(crow + 8 * p);
    cw[0] = c8.x;
    cw[1] = c8.y;
  }
  __builtin_amdgcn_wave_barrier();
  float kv[CL];
  int bj[CL];
#pragma unroll
  for (int e = 0; e < CL; ++e) {
    bj[e] = (int)((cw[e >> 2] >> (8 * (e & 3))) & 0xffu);  // stale past the total: unused
    const float x = srow[gate_col(bj[e])];
    kv[e] = CL * p + e < total ? x : -INFINITY;
  }
  float t = ninf;  // -inf: every candidate is selected
  if (__ballot(rv && total != k1) != 0ull) {
    float sk[CL];
#pragma unroll
    for (int e = 0; e < CL; ++e) sk[e] = kv[e];
    group_sort_asc<CL>(sk, p, pinf, ninf);
    t = group_pick<CL>(sk, kCap - k1, lane);
  }
  int cg = 0, ce = 0;
  bool gt[CL], eq[CL];
#pragma unroll
  for (int e = 0; e < CL; ++e) {
    const bool real = CL * p + e < total;
    gt[e] = real && kv[e] > t;
    eq[e] = real && kv[e] == t;
    cg += gt[e];
    ce += eq[e];
  }
  int gt_before, eq_before, sel_before;
  const int ngt = group_scan(cg, p, &gt_before);
  group_scan(ce, p, &eq_before);
  const int need = k1 - ngt;  // candidates equal to t to take, lowest block ids first
  bool sel[CL];
  int cs = 0, run = eq_before;
#pragma unroll
  for (int e = 0; e < CL; ++e) {
    sel[e] = gt[e] || (eq[e] && run < need);
    run += eq[e];
    cs += sel[e];
  }
  const int nsel = group_scan(cs, p, &sel_before);
  if (rv) {
    int32_t* orow = rows0 + (size_t)r * row_stride;
    int o = sel_before;
#pragma unroll
    for (int e = 0; e < CL; ++e)
      if (sel[e]) orow[o++] = bj[e];
    for (int qq = nsel + p; qq < topk; qq += 8) orow[qq] = qq == nsel ? c : -1;
  }
  return true;
}

// Rows of one wave whose candidate selection gave up, one row at a time over
// the whole wave (lane l holds the keys of blocks l, l + 64, ...): a bitwise
// radix select of the (k - 1)-th largest order key, then every key above it
// plus the lowest-index keys equal to it.  Slow but indifferent to ties.
__device__ __noinline__ void gate_select_rows(const float (*ss)[kGateStride], int w, int lane,
                                              int nq, int nspan, int k1, int topk, int c,
                                              int32_t* rows0, int row_stride) {
  for (int rr = 0; rr < kGateRowsPerWave; ++rr) {
    const int r = w * kGateRowsPerWave + rr;
    if (r >= nq) break;
    uint32_t key[4];
    int total = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j = lane + 64 * q;
      key[q] = j < nspan ? order_key(ss[r][gate_col(j)]) : 0u;
      total += (int)__popcll(__ballot(key[q] != 0u));
    }
    uint32_t thr = 0u;  // 0: at most k1 keys, all of them taken
    if (total > k1) {
      for (int b = 31; b >= 0; --b) {
        const uint32_t cnd = thr | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) cnt += (int)__popcll(__ballot(key[q] >= cnd));
        if (cnt >= k1) {
          thr = cnd;
          if (cnt == k1) break;  // the k1 keys >= thr are the selection
        }
      }
    }
    int need = k1;
#pragma unroll
    for (int q = 0; q < 4; ++q) need -= (int)__popcll(__ballot(key[q] > thr));
    int32_t* orow = rows0 + (size_t)r * row_stride;
    int pos = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint64_t em = __ballot(thr != 0u && key[q] == thr);
      const bool sel = key[q] > thr || (thr != 0u && key[q] == thr && lanes_below(em) < need);
      need -= min(need, (int)__popcll(em));
      const uint64_t m = __ballot(sel);
      if (sel) orow[pos + lanes_below(m)] = lane + 64 * q;
      pos += (int)__popcll(m);
    }
    for (int qq = pos + lane; qq < topk; qq += 64) orow[qq] = qq == pos ? c : -1;
  }
}

// One workgroup (8 waves, two per CU) handles 64 consecutive query tokens
// of one sequence and head (B is a multiple of 64, so they share their own
// block c) whose past blocks fit one span (c <= 256): they are scored into LDS, then each wave selects for its 8 rows
// with the candidate selection (k - 1 <= kSelMaxK), or row by row when that
// gives up.  Among keys equal to the threshold the lower block indices win.
template <typename T, int D, bool QUEST>
__global__ __launch_bounds__(kSpanWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void gate_span_kernel(
    const T* __restrict__ q, const float* __restrict__ kbar, const uint16_t* __restrict__ kbar3,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ cu_blocks,
    int total_tokens, int total_blocks, int tiles_per_seq, int H, int block_size, int topk,
    int32_t* __restrict__ block_idx) {
  constexpr bool kMfma = sizeof(T) == 2;
  static_assert(kMfma || !QUEST, "the min/max pooled gate runs on the bf16 path");
  __shared__ __attribute__((aligned(16))) float ss[kSpanRows][kGateStride];
  __shared__ __attribute__((aligned(16))) uint8_t cand[kSpanWaves][kGateRowsPerWave][kSelCap];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int sid = blockIdx.x / tiles_per_seq;
  const int tile = tiles_per_seq - 1 - (blockIdx.x % tiles_per_seq);  // heavy tiles first
  const int h = blockIdx.y;
  int start, len;
  seq_span(cu_seqlens, sid, total_tokens, &start, &len);
  const int p0 = tile * kSpanRows;
  if (p0 >= len) return;
  const int c = p0 / block_size;
  if (c > kGateSpan) return;  // several spans: gate_topk_kernel
  const int nq = min(kSpanRows, len - p0);
  const int k1 = topk - 1;
  const int gb0 = cu_blocks[sid];
  int32_t* rows0 = block_idx + ((size_t)(start + p0) * H + h) * topk;
  const int rs = H * topk;
  if (c <= k1 || k1 == 0) {
    // no choice: every past block (c <= k - 1) or none (k = 1), then the own
    // block, then -1
    for (int i = tid; i < nq * topk; i += kSpanWaves * 64) {
      const int r = i / topk, j = i - r * topk;
      rows0[(size_t)r * rs + j] = k1 == 0 ? (j == 0 ? c : -1) : (j <= c ? j : -1);
    }
    return;
  }
  if constexpr (kMfma) {
    static_assert(32 * kSpanWaves == kGateSpan, "one 32-block tile per wave covers the span");
    if (32 * w < c) {
      if constexpr (QUEST)
        gate_scores_span_minmax<D>((const uint16_t*)q, start, len, p0, H, h, kbar, gb0, c,
                                   total_blocks, ss, w, lane);
      else
        gate_scores_span<D>((const uint16_t*)q, start, len, p0, H, h, kbar3, gb0, c,
                            total_blocks, ss, w, lane);
    }
    __syncthreads();
  } else {
    __shared__ __attribute__((aligned(16))) float qs[kSpanRows][D + 4];
    __shared__ __attribute__((aligned(16))) float ks[kGateChunkValu][D + 4];
    for (int i = tid; i < kSpanRows * (D / 4); i += kSpanWaves * 64) {
      const int r = i / (D / 4), e4 = i % (D / 4);
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (r < nq)
        v = *reinterpret_cast<const f32x4*>((const float*)q + ((size_t)(start + p0 + r) * H + h) * D + e4 * 4);
      *reinterpret_cast<f32x4*>(&qs[r][e4 * 4]) = v;
    }
    for (int cb = 0; cb < c; cb += kGateChunkValu)
      gate_scores_valu<D, kSpanWaves * 64>(qs, ks, kbar, H, h, gb0 + cb, min(kGateChunkValu, c - cb),
                          total_blocks, ss, cb, tid);
  }
  bool done = false;
  if (k1 <= 4)
    done = gate_select_candidates<1, 4>(ss, cand[w], w, lane, nq, c, k1, topk, c, rows0, rs);
  else if (k1 <= 11)
    done = gate_select_candidates<2, 4>(ss, cand[w], w, lane, nq, c, k1, topk, c, rows0, rs);
  else if (k1 <= 24)
    done = gate_select_candidates<4, 4>(ss, cand[w], w, lane, nq, c, k1, topk, c, rows0, rs);
  else if (k1 <= kSelMaxK)
    done = gate_select_candidates<8, 8>(ss, cand[w], w, lane, nq, c, k1, topk, c, rows0, rs);
  if (!done) gate_select_rows(ss, w, lane, nq, c, k1, topk, c, rows0, rs);
}

// Tiles whose past blocks span several 256-block spans (and, with skip_span
// 0, every tile): one workgroup per 32 query tokens of one sequence and head
// as above; the past blocks are scored into LDS 256 at a time and each span
// is merged into a kept set of at most k - 1 keys per row (see the selection
// paths below); among keys equal to the threshold the lower block indices
// win.
template <typename T, int D, bool QUEST>
__global__ __launch_bounds__(kGateWaves * 64) __attribute__((amdgpu_waves_per_eu(QUEST || D > 64 ? 2 : 4))) void gate_topk_kernel(
    const T* __restrict__ q, const float* __restrict__ kbar, const uint16_t* __restrict__ kbar3,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ cu_blocks,
    int total_tokens, int total_blocks, int tiles_per_seq, int H, int block_size, int topk,
    int skip_span, int32_t* __restrict__ block_idx) {
  constexpr bool kMfma = sizeof(T) == 2;
  static_assert(kMfma || !QUEST, "the min/max pooled gate runs on the bf16 path");
  __shared__ __attribute__((aligned(16))) float ss[kGateRows][kGateStride];
  __shared__ uint32_t skey[kGateWaves][64];
  __shared__ int32_t sidx[kGateWaves][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int sid = blockIdx.x / tiles_per_seq;
  const int tile = tiles_per_seq - 1 - (blockIdx.x % tiles_per_seq);  // heavy tiles first
  const int h = blockIdx.y;
  int start, len;
  seq_span(cu_seqlens, sid, total_tokens, &start, &len);
  const int p0 = tile * kGateRows;
  if (p0 >= len) return;
  const int nq = min(kGateRows, len - p0);
  const int c = p0 / block_size;
  if (skip_span && c <= kGateSpan) return;  // gate_span_kernel
  const int k1 = topk - 1;
  const int gb0 = cu_blocks[sid];
  if (c <= k1) {
    // at most k - 1 past blocks: all of them are selected, so the rows need
    // no scores (blocks 0 .. c ascending, the own block last, then -1)
    for (int i = tid; i < nq * topk; i += kGateWaves * 64) {
      const int r = i / topk, j = i - r * topk;
      block_idx[((size_t)(start + p0 + r) * H + h) * topk + j] = j <= c ? j : -1;
    }
    return;
  }

  uint32_t tkey[kGateRowsPerWave];
  int32_t tidx[kGateRowsPerWave];
  int tcnt[kGateRowsPerWave];
#pragma unroll
  for (int i = 0; i < kGateRowsPerWave; ++i) { tkey[i] = 0u; tidx[i] = -1; tcnt[i] = 0; }

  if (k1 > 0 && c > 0) {
    // query operands: bf16 MFMA fragments in registers, or an fp32 LDS tile
    bf16x8 qfrag[D / 16];
    if constexpr (kMfma) {
      const int tok = p0 + 32 * (w >> 2) + (lane & 31);
      const bool qv = tok < len;
      const uint16_t* qp = (const uint16_t*)q + ((size_t)(start + (qv ? tok : p0)) * H + h) * D +
                           8 * (lane >> 5);
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        u32x4 wv = {0u, 0u, 0u, 0u};
        if (qv) wv = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
        qfrag[ks] = __builtin_bit_cast(bf16x8, wv);
      }
    }
    for (int base = 0; base < c; base += kGateSpan) {
      const int nspan = min(kGateSpan, c - base);
      if constexpr (kMfma) {
        for (int cb = 0; cb < nspan; cb += kGateChunk) {
          if constexpr (QUEST)
            gate_scores_mfma<D, true>(qfrag, kbar, H, h, gb0 + base + cb,
                                      min(kGateChunk, nspan - cb), total_blocks, ss, cb, w, lane);
          else
            gate_scores_planes<D>(qfrag, kbar3, H, h, gb0 + base + cb,
                                  min(kGateChunk, nspan - cb), total_blocks, ss, cb, w, lane);
        }
        __syncthreads();
      } else {
        __shared__ __attribute__((aligned(16))) float qs[kGateRows][D + 4];
        __shared__ __attribute__((aligned(16))) float ks[kGateChunkValu][D + 4];
        if (base == 0) {
          for (int i = tid; i < kGateRows * (D / 4); i += kGateWaves * 64) {
            const int r = i / (D / 4), e4 = i % (D / 4);
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            if (r < nq)
              v = *reinterpret_cast<const f32x4*>((const float*)q + ((size_t)(start + p0 + r) * H + h) * D + e4 * 4);
            *reinterpret_cast<f32x4*>(&qs[r][e4 * 4]) = v;
          }
        }
        for (int cb = 0; cb < nspan; cb += kGateChunkValu)
          gate_scores_valu<D, kGateWaves * 64>(qs, ks, kbar, H, h, gb0 + base + cb,
                              min(kGateChunkValu, nspan - cb), total_blocks, ss, cb, tid);
      }

      // The wave's 8 rows go through the radix select in lockstep (independent
      // dependency chains).  Order keys of finite scores are >= 1, so key 0
      // marks "no candidate" (lanes past the span, rows past the tile end,
      // unused slots of the kept set) and never reaches a threshold >= 1.
      constexpr int R = kGateRowsPerWave;
      uint32_t prefix[R];
      if (k1 <= kGateFastK) {
        // Threshold = the k1-th largest key of the row, found with VALU work
        // only: lane (row lane / 8, part lane % 8) keeps the sorted
        // (descending) top 16 of the row's keys j = part, part + 8, ...
        // (branch-free max/min insertion), the 8 parts are merged in three
        // xor-shuffle rounds (the half-cleaner max(a_i, b_15-i) keeps the top
        // 16 of both lists as a bitonic sequence, which a bitonic merge sorts).
        const int rr = lane >> 3, part = lane & 7;
        const int r = w * R + rr;
        uint32_t top[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) top[i] = 0u;
        auto insert = [&](uint32_t x) {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const uint32_t hi = max(top[i], x);
            x = min(top[i], x);
            top[i] = hi;
          }
        };
        if (r < nq)
          for (int j = part; j < nspan; j += 8) insert(order_key(ss[r][gate_col(j)]));
        if (base > 0) {
          // the row's kept set (at most k1 <= 16 keys, lanes 0..15 of the
          // row-per-wave layout)
          uint32_t a0 = 0u, a1 = 0u;
#pragma unroll
          for (int i = 0; i < R; ++i) {
            const uint32_t b0 = __shfl(tkey[i], part), b1 = __shfl(tkey[i], part + 8);
            if (rr == i) { a0 = b0; a1 = b1; }
          }
          insert(a0);
          insert(a1);
        }
#pragma unroll
        for (int d = 1; d < 8; d <<= 1) {
          uint32_t pt[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) pt[i] = __shfl_xor(top[i], d);
#pragma unroll
          for (int i = 0; i < 16; ++i) top[i] = max(top[i], pt[15 - i]);
#pragma unroll
          for (int dist = 8; dist >= 1; dist >>= 1)
#pragma unroll
            for (int i = 0; i < 16; ++i)
              if ((i & dist) == 0) {
                const uint32_t hi = max(top[i], top[i + dist]);
                const uint32_t lo = min(top[i], top[i + dist]);
                top[i] = hi;
                top[i + dist] = lo;
              }
        }
        // 0 when the row has fewer than k1 candidates: all of them are kept
        uint32_t t = 0u;
#pragma unroll
        for (int i = 0; i < 16; ++i) t = (i == k1 - 1) ? top[i] : t;
#pragma unroll
        for (int i = 0; i < R; ++i) prefix[i] = __builtin_amdgcn_readlane(t, 8 * i);
      }
      uint32_t nkey[R][4];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int r = w * R + i;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          nkey[i][j] = (r < nq && lane + 64 * j < nspan) ? order_key(ss[r][gate_col(lane + 64 * j)]) : 0u;
      }
      if (k1 > kGateFastK) {
      // Bitwise radix select of the k1-th largest key, most significant bit
      // first.  A row is settled as soon as exactly k1 keys reach the
      // candidate prefix (they are the selection, whatever the lower bits),
      // or from the start when it has at most k1 candidates (prefix 0 keeps
      // them all).  Groups of 64 past the span and an empty kept set hold
      // only key 0 and are not counted.
      const int ngrp = (nspan + 63) / 64;
      bool done[R];
#pragma unroll
      for (int i = 0; i < R; ++i) {
        prefix[i] = 0u;
        int total = tcnt[i];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (j < ngrp) total += (int)__popcll(__ballot(nkey[i][j] != 0u));
        done[i] = total <= k1;
      }
      for (int b = 31; b >= 0; --b) {
        bool all = true;
#pragma unroll
        for (int i = 0; i < R; ++i) {
          if (!done[i]) {
            const uint32_t cand = prefix[i] | (1u << b);
            int cnt = tcnt[i] > 0 ? (int)__popcll(__ballot(tkey[i] >= cand)) : 0;
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (j < ngrp) cnt += (int)__popcll(__ballot(nkey[i][j] >= cand));
            if (cnt >= k1) {
              prefix[i] = cand;
              done[i] = cnt == k1;
            }
          }
          all = all && done[i];
        }
        if (all) break;
      }
      }
#pragma unroll
      for (int i = 0; i < R; ++i) {
        // thr = 0 when there are at most k1 candidates: all of them are kept
        const uint32_t thr = prefix[i];
        int need = k1 - (int)__popcll(__ballot(tkey[i] > thr));
#pragma unroll
        for (int j = 0; j < 4; ++j) need -= (int)__popcll(__ballot(nkey[i][j] > thr));
        // keys equal to the threshold: lowest block index first (old set, then new)
        const uint64_t eo = __ballot(thr != 0u && tkey[i] == thr);
        const bool so = tkey[i] > thr || (thr != 0u && tkey[i] == thr && lanes_below(eo) < need);
        need -= min(need, (int)__popcll(eo));
        bool sn[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint64_t en = __ballot(thr != 0u && nkey[i][j] == thr);
          sn[j] = nkey[i][j] > thr || (thr != 0u && nkey[i][j] == thr && lanes_below(en) < need);
          need -= min(need, (int)__popcll(en));
        }
        // compact: kept old entries, then new ones in block order
        const uint64_t mo = __ballot(so);
        int pos0 = (int)__popcll(mo);
        __builtin_amdgcn_wave_barrier();
        if (so) { skey[w][lanes_below(mo)] = tkey[i]; sidx[w][lanes_below(mo)] = tidx[i]; }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint64_t mn = __ballot(sn[j]);
          if (sn[j]) {
            const int pos = pos0 + lanes_below(mn);
            skey[w][pos] = nkey[i][j];
            sidx[w][pos] = base + lane + 64 * j;
          }
          pos0 += (int)__popcll(mn);
        }
        __builtin_amdgcn_wave_barrier();
        tkey[i] = lane < pos0 ? skey[w][lane] : 0u;
        tidx[i] = lane < pos0 ? sidx[w][lane] : -1;
        tcnt[i] = pos0;
        __builtin_amdgcn_wave_barrier();
      }
      // the scores are overwritten by the next span (a single span needs no
      // barrier: waves may have left through the paths above)
      if (base + kGateSpan < c) __syncthreads();
    }
  }

  // Rows: the kept past blocks (ascending), then the own block, then -1.
#pragma unroll
  for (int i = 0; i < kGateRowsPerWave; ++i) {
    const int r = w * kGateRowsPerWave + i;
    if (r >= nq) continue;
    if (lane < topk) {
      int v;
      if (lane < tcnt[i]) v = tidx[i];
      else if (lane == tcnt[i]) v = c;
      else v = -1;
      block_idx[((size_t)(start + p0 + r) * H + h) * topk + lane] = v;
    }
  }
}

// ---------------------------------------------------------------------------
// static routing: fixed gates (sliding window, sink + window, full attention)
// ---------------------------------------------------------------------------
// Row of a query whose own block is c, as a closed form: with every block
// taken when c < topk, else the s = min(sink, topk - 1) initial blocks and
// the topk - s most recent blocks c - (topk - 1 - s) .. c, ascending.
constexpr int kStaticTokens = 64;  // tokens per workgroup

__global__ __launch_bounds__(256) void static_select_kernel(
    const int32_t* __restrict__ cu_seqlens, int total_tokens, int tiles, int H, int block_size,
    int topk, int sink, int32_t* __restrict__ block_idx) {
  const int s = blockIdx.x / tiles;
  const int p0 = (blockIdx.x - s * tiles) * kStaticTokens;
  int start, len;
  seq_span(cu_seqlens, s, total_tokens, &start, &len);
  if (p0 >= len) return;
  const int n = min(kStaticTokens, len - p0);
  const int sk = min(sink, topk - 1);
  // one thread per (token, head) row; consecutive threads write consecutive rows
  for (int r = threadIdx.x; r < n * H; r += blockDim.x) {
    const int tok = r / H;
    const int c = (p0 + tok) / block_size;
    const int lo = c - (topk - 1 - sk);  // first recent block when c >= topk
    int32_t* row = block_idx + ((size_t)(start + p0) * H + r) * topk;
    auto value = [&](int j) {
      if (c < topk) return j <= c ? j : -1;
      return j < sk ? j : lo + (j - sk);
    };
    if ((topk & 3) == 0) {  // rows start 16-byte aligned
      for (int j = 0; j < topk; j += 4)
        *reinterpret_cast<int4*>(row + j) = make_int4(value(j), value(j + 1), value(j + 2),
                                                      value(j + 3));
    } else {
      for (int j = 0; j < topk; ++j) row[j] = value(j);
    }
  }
}

// ---------------------------------------------------------------------------
// launches
// ---------------------------------------------------------------------------
hipError_t launch_pool_keys(const void* k, bool bf16, const Geo& g, float* kbar,
                            uint16_t* kbar3, hipStream_t st) {
  if (g.total_blocks == 0) return hipSuccess;
  const int hd = g.num_heads * g.head_dim;
  dim3 grid(g.total_blocks, hd / 64);
  if (bf16)
    hipLaunchKernelGGL(pool_keys_kernel<uint16_t>, grid, dim3(256), 0, st,
                       (const uint16_t*)k, g.cu_seqlens, g.cu_blocks, g.num_seqs,
                       g.total_tokens, hd, g.head_dim, g.block_size, kbar, kbar3);
  else
    hipLaunchKernelGGL(pool_keys_kernel<float>, grid, dim3(256), 0, st, (const float*)k,
                       g.cu_seqlens, g.cu_blocks, g.num_seqs, g.total_tokens, hd, g.head_dim,
                       g.block_size, kbar, kbar3);
  return hipGetLastError();
}

hipError_t launch_pool_minmax(const void* k, bool bf16, const Geo& g, float* kmm,
                              hipStream_t st) {
  if (g.total_blocks == 0) return hipSuccess;
  const int hd = g.num_heads * g.head_dim;
  dim3 grid(g.total_blocks, hd / 64);
  if (bf16)
    hipLaunchKernelGGL(pool_minmax_kernel<uint16_t>, grid, dim3(256), 0, st,
                       (const uint16_t*)k, g.cu_seqlens, g.cu_blocks, g.num_seqs,
                       g.total_tokens, g.total_blocks, hd, g.head_dim, g.block_size, kmm);
  else
    hipLaunchKernelGGL(pool_minmax_kernel<float>, grid, dim3(256), 0, st, (const float*)k,
                       g.cu_seqlens, g.cu_blocks, g.num_seqs, g.total_tokens, g.total_blocks,
                       hd, g.head_dim, g.block_size, kmm);
  return hipGetLastError();
}

// The span kernel takes every tile with at most 256 past blocks when
// k - 1 <= kSelMaxK; gate_topk_kernel takes the rest (launched only when
// there is a rest).
template <typename T, int D, bool QUEST>
void launch_gate(const T* q, const float* kbar, const uint16_t* kbar3, const Geo& g, int topk,
                 int32_t* block_idx, hipStream_t st) {
  const int tiles = (g.max_seqlen + kGateRows - 1) / kGateRows;
  dim3 grid(g.num_seqs * tiles, g.num_heads);
  dim3 block(kGateWaves * 64);
  const bool span = topk - 1 <= kSelMaxK;
  const int c_max = (g.max_seqlen - 1) / kGateRows * kGateRows / g.block_size;
  if (span) {
    const int stiles = (g.max_seqlen + kSpanRows - 1) / kSpanRows;
    hipLaunchKernelGGL((gate_span_kernel<T, D, QUEST>), dim3(g.num_seqs * stiles, g.num_heads),
                       dim3(kSpanWaves * 64), 0, st, q, kbar, kbar3, g.cu_seqlens, g.cu_blocks,
                       g.total_tokens, g.total_blocks, stiles, g.num_heads, g.block_size, topk,
                       block_idx);
  }
  if (!span || c_max > kGateSpan)
    hipLaunchKernelGGL((gate_topk_kernel<T, D, QUEST>), grid, block, 0, st, q, kbar, kbar3,
                       g.cu_seqlens, g.cu_blocks, g.total_tokens, g.total_blocks, tiles,
                       g.num_heads, g.block_size, topk, span ? 1 : 0, block_idx);
}

hipError_t launch_gate_topk_minmax(const uint16_t* q, const float* kmm, const Geo& g, int topk,
                                   int32_t* block_idx, hipStream_t st) {
  if (g.total_tokens == 0 || g.max_seqlen == 0) return hipSuccess;
  if (g.head_dim == 128) launch_gate<uint16_t, 128, true>(q, kmm, nullptr, g, topk, block_idx, st);
  else launch_gate<uint16_t, 64, true>(q, kmm, nullptr, g, topk, block_idx, st);
  return hipGetLastError();
}

hipError_t launch_gate_topk(const void* q, bool bf16, const float* kbar, const uint16_t* kbar3,
                            const Geo& g, int topk, int32_t* block_idx, hipStream_t st) {
  if (g.total_tokens == 0 || g.max_seqlen == 0) return hipSuccess;
  if (bf16) {
    const uint16_t* qb = (const uint16_t*)q;
    if (g.head_dim == 128) launch_gate<uint16_t, 128, false>(qb, kbar, kbar3, g, topk, block_idx, st);
    else launch_gate<uint16_t, 64, false>(qb, kbar, kbar3, g, topk, block_idx, st);
  } else {
    const float* qf = (const float*)q;
    if (g.head_dim == 128) launch_gate<float, 128, false>(qf, kbar, kbar3, g, topk, block_idx, st);
    else launch_gate<float, 64, false>(qf, kbar, kbar3, g, topk, block_idx, st);
  }
  return hipGetLastError();
}

hipError_t launch_static_select(const Geo& g, int topk, int sink, int32_t* block_idx,
                                hipStream_t st) {
  if (g.total_tokens == 0 || g.max_seqlen == 0) return hipSuccess;
  const int tiles = (g.max_seqlen + kStaticTokens - 1) / kStaticTokens;
  hipLaunchKernelGGL(static_select_kernel, dim3(g.num_seqs * tiles), dim3(256), 0, st,
                     g.cu_seqlens, g.total_tokens, tiles, g.num_heads, g.block_size, topk, sink,
                     block_idx);
  return hipGetLastError();
}

}  // namespace moba
