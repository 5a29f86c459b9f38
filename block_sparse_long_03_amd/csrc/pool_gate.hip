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

template <typename T>
__global__ __launch_bounds__(256) void pool_keys_kernel(
    const T* __restrict__ k, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ cu_blocks, int num_seqs, int total_tokens, int hd,
    int block_size, float* __restrict__ kbar) {
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
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = cnt > 0 ? red[0][tx * 8 + i] / inv_cnt : 0.f;
  }
}

// min/max pool: kmm[gb, h, 0, :] = elementwise max of the block's keys,
// kmm[gb, h, 1, :] = elementwise min (exact: no rounding)
template <typename T>
__global__ __launch_bounds__(256) void pool_minmax_kernel(
    const T* __restrict__ k, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ cu_blocks, int num_seqs, int total_tokens, int hd, int D,
    int block_size, float* __restrict__ kmm) {
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
    // column col0 + 8 tx + i of the [H * D] row is (head, dim) = divmod(col, D)
    const int col = col0 + tx * 8;
    const int h = col / D, e = col - h * D;
    float* dst = kmm + ((size_t)gb * (hd / D) + h) * 2 * D + e;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      dst[i] = cnt > 0 ? rmax[0][tx * 8 + i] : 0.f;
      dst[D + i] = cnt > 0 ? rmin[0][tx * 8 + i] : 0.f;
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
constexpr int kGateStride = kGateSpan + 8;  // LDS row stride of the scores (8 banks apart)
constexpr int kGateFastK = 16;   // k - 1 up to this: threshold from sorted per-lane lists
constexpr int kGateChunk = 128;  // past blocks per MFMA scoring step (one 32 x 32 tile per wave)
constexpr int kGateChunkValu = 64;  // past blocks per fp32 scoring step
constexpr int kGateWaves = 4;
constexpr int kGateRowsPerWave = kGateRows / kGateWaves;

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
  const float* kp = kbar + ((size_t)(ok ? gblk0 + j : gblk0) * H + h) * KD + 8 * hf;
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  constexpr int KH = D / 32;  // k-steps per group (loads of a group in flight together)
#pragma unroll
  for (int half = 0; half < KD / (16 * KH); ++half) {
  f32x4 xa[KH], xb[KH];
#pragma unroll
  for (int kk = 0; kk < KH; ++kk) {
    xa[kk] = *reinterpret_cast<const f32x4*>(kp + 16 * (half * KH + kk));
    xb[kk] = *reinterpret_cast<const f32x4*>(kp + 16 * (half * KH + kk) + 4);
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
  for (int r = 0; r < 16; ++r)
    ss[32 * tt + l32][col0 + 32 * bt + 8 * (r >> 2) + 4 * hf + (r & 3)] = acc[r];
}

// fp32 queries: plain fp32 FMA over d in index order (LDS tiles of q and kbar)
template <int D>
__device__ __forceinline__ void gate_scores_valu(const float (*qs)[D + 4], float (*ks)[D + 4],
                                                 const float* __restrict__ kbar, int H, int h,
                                                 int gblk0, int nb, int total_blocks,
                                                 float (*ss)[kGateStride], int col0, int tid) {
  for (int i = tid; i < kGateChunkValu * (D / 4); i += kGateWaves * 64) {
    const int j = i / (D / 4), e4 = i % (D / 4);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (j < nb && gblk0 + j < total_blocks)
      v = *reinterpret_cast<const f32x4*>(kbar + ((size_t)(gblk0 + j) * H + h) * D + e4 * 4);
    *reinterpret_cast<f32x4*>(&ks[j][e4 * 4]) = v;
  }
  __syncthreads();
  const int ty = tid >> 4;  // rows 2ty, 2ty+1
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
    ss[2 * ty][col0 + tx + 16 * jj] = acc[0][jj];
    ss[2 * ty + 1][col0 + tx + 16 * jj] = acc[1][jj];
  }
  __syncthreads();  // ks is reused by the next chunk
}

// One workgroup (4 waves, small enough for four per CU) handles 32
// consecutive query tokens of one sequence and head (B is a multiple of 64,
// so they share their own block c).  The past blocks are scored into LDS up
// to 256 at a time; each wave then selects for its 8 rows (see the two
// selection paths below); among keys equal to the threshold the lower block
// indices win.
template <typename T, int D, bool QUEST>
__global__ __launch_bounds__(kGateWaves * 64) __attribute__((amdgpu_waves_per_eu(QUEST && D > 64 ? 2 : 4))) void gate_topk_kernel(
    const T* __restrict__ q, const float* __restrict__ kbar,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ cu_blocks,
    int total_tokens, int total_blocks, int tiles_per_seq, int H, int block_size, int topk,
    int32_t* __restrict__ block_idx) {
  constexpr bool kMfma = sizeof(T) == 2;
  static_assert(kMfma || !QUEST, "the min/max pooled gate runs on the bf16 path");
  __shared__ float ss[kGateRows][kGateStride];
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
        for (int cb = 0; cb < nspan; cb += kGateChunk)
          gate_scores_mfma<D, QUEST>(qfrag, kbar, H, h, gb0 + base + cb, min(kGateChunk, nspan - cb),
                              total_blocks, ss, cb, w, lane);
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
          gate_scores_valu<D>(qs, ks, kbar, H, h, gb0 + base + cb,
                              min(kGateChunkValu, nspan - cb), total_blocks, ss, cb, tid);
      }

      // The wave's 8 rows go through the radix select in lockstep (independent
      // dependency chains).  Order keys of finite scores are >= 1, so key 0
      // marks "no candidate" (lanes past the span, rows past the tile end,
      // unused slots of the kept set) and never reaches a threshold >= 1.
      constexpr int R = kGateRowsPerWave;
      if (c <= kGateSpan && k1 <= kGateFastK) {
        // Single span, k1 <= 16: the whole selection in the 8-lanes-per-row
        // layout, VALU only.  The threshold is the k1-th largest key (sorted
        // per-lane top 16, bitonic merges); lane (row lane / 8, part
        // lane % 8) then owns the candidates j = 32 part + m, m < 32 (its
        // 32-bit word of the row's bitmap): the selection is every key above
        // the threshold plus the lowest-index keys equal to it, written in
        // ascending order.
        const int rr = lane >> 3, part = lane & 7;
        const int r = w * R + rr;
        const bool rv = r < nq;
        auto key_at = [&](int m) {
          const int j = 32 * part + m;
          return (rv && j < nspan) ? order_key(ss[r][j]) : 0u;
        };
        uint32_t top[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) top[i] = 0u;
        // the threshold pass takes the row's keys strided (j = part + 8 m),
        // so each lane inserts only ceil(nspan / 8) of them; the 8 parts of a
        // row sit in distinct banks (row stride 8 banks)
        for (int j = part; j < nspan; j += 8) {
          uint32_t x = rv ? order_key(ss[r][j]) : 0u;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const uint32_t hi = max(top[i], x);
            x = min(top[i], x);
            top[i] = hi;
          }
        }
        const int nm = min(32, nspan);
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
        uint32_t t = 0u;  // 0: fewer than k1 candidates, all of them are kept
#pragma unroll
        for (int i = 0; i < 16; ++i) t = (i == k1 - 1) ? top[i] : t;
        uint32_t gt = 0u, eq = 0u;
        for (int mm = 0; mm < nm; ++mm) {
          const int m = (mm + part) & 31;
          const uint32_t x = key_at(m);
          gt |= (uint32_t)(x > t && x != 0u) << m;
          eq |= (uint32_t)(t != 0u && x == t) << m;
        }
        // sums and exclusive prefixes over the 8 parts of a row
        auto row_scan = [&](int v, int& excl) {
          int inc = v;
#pragma unroll
          for (int d = 1; d < 8; d <<= 1) {
            const int u = __shfl_up(inc, d, 8);
            if (part >= d) inc += u;
          }
          excl = inc - v;
          return __shfl(inc, 7, 8);
        };
        int gt_before, eq_before, sel_before;
        const int ngt = row_scan(__popc(gt), gt_before);
        row_scan(__popc(eq), eq_before);
        // keys equal to the threshold: lowest block indices first
        int take = min(max(k1 - ngt - eq_before, 0), __popc(eq));
        uint32_t sel = gt, e = eq;
        for (; take > 0; --take) {
          sel |= e & (~e + 1u);
          e &= e - 1u;
        }
        const int nsel = row_scan(__popc(sel), sel_before);
        if (rv) {
          int32_t* out = block_idx + ((size_t)(start + p0 + r) * H + h) * topk;
          int pos = sel_before;
          for (uint32_t sm = sel; sm != 0u; sm &= sm - 1u)
            out[pos++] = base + 32 * part + __builtin_ctz(sm);
          for (int q = nsel + part; q < topk; q += 8) out[q] = q == nsel ? c : -1;
        }
        return;
      }
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
          for (int j = part; j < nspan; j += 8) insert(order_key(ss[r][j]));
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
          nkey[i][j] = (r < nq && lane + 64 * j < nspan) ? order_key(ss[r][lane + 64 * j]) : 0u;
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
      __syncthreads();
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
                            hipStream_t st) {
  if (g.total_blocks == 0) return hipSuccess;
  const int hd = g.num_heads * g.head_dim;
  dim3 grid(g.total_blocks, hd / 64);
  if (bf16)
    hipLaunchKernelGGL(pool_keys_kernel<uint16_t>, grid, dim3(256), 0, st,
                       (const uint16_t*)k, g.cu_seqlens, g.cu_blocks, g.num_seqs,
                       g.total_tokens, hd, g.block_size, kbar);
  else
    hipLaunchKernelGGL(pool_keys_kernel<float>, grid, dim3(256), 0, st, (const float*)k,
                       g.cu_seqlens, g.cu_blocks, g.num_seqs, g.total_tokens, hd,
                       g.block_size, kbar);
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
                       g.total_tokens, hd, g.head_dim, g.block_size, kmm);
  else
    hipLaunchKernelGGL(pool_minmax_kernel<float>, grid, dim3(256), 0, st, (const float*)k,
                       g.cu_seqlens, g.cu_blocks, g.num_seqs, g.total_tokens, hd, g.head_dim,
                       g.block_size, kmm);
  return hipGetLastError();
}

hipError_t launch_gate_topk_minmax(const uint16_t* q, const float* kmm, const Geo& g, int topk,
                                   int32_t* block_idx, hipStream_t st) {
  if (g.total_tokens == 0 || g.max_seqlen == 0) return hipSuccess;
  const int tiles = (g.max_seqlen + kGateRows - 1) / kGateRows;
  dim3 grid(g.num_seqs * tiles, g.num_heads);
  dim3 block(kGateWaves * 64);
  if (g.head_dim == 128)
    hipLaunchKernelGGL((gate_topk_kernel<uint16_t, 128, true>), grid, block, 0, st, q, kmm,
                       g.cu_seqlens, g.cu_blocks, g.total_tokens, g.total_blocks, tiles,
                       g.num_heads, g.block_size, topk, block_idx);
  else
    hipLaunchKernelGGL((gate_topk_kernel<uint16_t, 64, true>), grid, block, 0, st, q, kmm,
                       g.cu_seqlens, g.cu_blocks, g.total_tokens, g.total_blocks, tiles,
                       g.num_heads, g.block_size, topk, block_idx);
  return hipGetLastError();
}

hipError_t launch_gate_topk(const void* q, bool bf16, const float* kbar, const Geo& g,
                            int topk, int32_t* block_idx, hipStream_t st) {
  if (g.total_tokens == 0 || g.max_seqlen == 0) return hipSuccess;
  const int tiles = (g.max_seqlen + kGateRows - 1) / kGateRows;
  dim3 grid(g.num_seqs * tiles, g.num_heads);
  dim3 block(kGateWaves * 64);
#define MOBA_GATE(T, D)                                                                   \
  hipLaunchKernelGGL((gate_topk_kernel<T, D, false>), grid, block, 0, st, (const T*)q, kbar, \
                     g.cu_seqlens, g.cu_blocks, g.total_tokens, g.total_blocks, tiles,    \
                     g.num_heads,                                                         \
                     g.block_size, topk, block_idx)
  if (bf16) {
    if (g.head_dim == 128) MOBA_GATE(uint16_t, 128); else MOBA_GATE(uint16_t, 64);
  } else {
    if (g.head_dim == 128) MOBA_GATE(float, 128); else MOBA_GATE(float, 64);
  }
#undef MOBA_GATE
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
