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

constexpr int kGateRows = 64;     // query tokens per workgroup (one block c)
constexpr int kGateChunk = 64;    // past blocks scored per pass
constexpr int kGateWaves = 8;
constexpr int kGateRowsPerWave = kGateRows / kGateWaves;

template <typename T, int D>
__device__ __forceinline__ void load_q_tile(const T* __restrict__ q, float (*qs)[D + 4],
                                            int tok0, int nq, int H, int h, int tid);

template <>
__device__ __forceinline__ void load_q_tile<uint16_t, 128>(const uint16_t* __restrict__ q,
                                                           float (*qs)[132], int tok0, int nq,
                                                           int H, int h, int tid) {
  for (int i = tid; i < kGateRows * 16; i += kGateWaves * 64) {
    int r = i >> 4, c = i & 15;
    float v[8];
    if (r < nq) load8<uint16_t>(q + ((size_t)(tok0 + r) * H + h) * 128 + c * 8, v);
    else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) qs[r][c * 8 + e] = v[e];
  }
}
template <>
__device__ __forceinline__ void load_q_tile<uint16_t, 64>(const uint16_t* __restrict__ q,
                                                          float (*qs)[68], int tok0, int nq,
                                                          int H, int h, int tid) {
  for (int i = tid; i < kGateRows * 8; i += kGateWaves * 64) {
    int r = i >> 3, c = i & 7;
    float v[8];
    if (r < nq) load8<uint16_t>(q + ((size_t)(tok0 + r) * H + h) * 64 + c * 8, v);
    else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) qs[r][c * 8 + e] = v[e];
  }
}
template <>
__device__ __forceinline__ void load_q_tile<float, 128>(const float* __restrict__ q,
                                                        float (*qs)[132], int tok0, int nq,
                                                        int H, int h, int tid) {
  for (int i = tid; i < kGateRows * 32; i += kGateWaves * 64) {
    int r = i >> 5, c = i & 31;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (r < nq) v = *reinterpret_cast<const f32x4*>(q + ((size_t)(tok0 + r) * H + h) * 128 + c * 4);
    *reinterpret_cast<f32x4*>(&qs[r][c * 4]) = v;
  }
}
template <>
__device__ __forceinline__ void load_q_tile<float, 64>(const float* __restrict__ q,
                                                       float (*qs)[68], int tok0, int nq,
                                                       int H, int h, int tid) {
  for (int i = tid; i < kGateRows * 16; i += kGateWaves * 64) {
    int r = i >> 4, c = i & 15;
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (r < nq) v = *reinterpret_cast<const f32x4*>(q + ((size_t)(tok0 + r) * H + h) * 64 + c * 4);
    *reinterpret_cast<f32x4*>(&qs[r][c * 4]) = v;
  }
}

// One workgroup handles 64 consecutive query tokens of one sequence and head.
// Since B is a multiple of 64 they share their own block c.  Past blocks are
// scored 64 at a time into LDS (fp32 FMA over d in index order); each wave
// then keeps, for each of its 8 rows, the running top-(k-1) set in lanes
// 0..k-2 (ascending block index).  Merging a chunk into the set is an exact
// radix select over 32-bit order keys (ballot counts), with ties on the
// threshold key given to the lower block index.
template <typename T, int D>
__global__ __launch_bounds__(512) void gate_topk_kernel(
    const T* __restrict__ q, const float* __restrict__ kbar,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ cu_blocks,
    int total_tokens, int total_blocks, int tiles_per_seq, int H, int block_size, int topk,
    int32_t* __restrict__ block_idx) {
  __shared__ __attribute__((aligned(16))) float qs[kGateRows][D + 4];
  __shared__ __attribute__((aligned(16))) float ks[kGateChunk][D + 4];
  __shared__ float ss[kGateRows][kGateChunk + 1];
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

  uint32_t tkey[kGateRowsPerWave];
  int32_t tidx[kGateRowsPerWave];
  int tcnt[kGateRowsPerWave];
#pragma unroll
  for (int i = 0; i < kGateRowsPerWave; ++i) { tkey[i] = 0u; tidx[i] = -1; tcnt[i] = 0; }

  if (k1 > 0 && c > 0) {
    load_q_tile<T, D>(q, qs, start + p0, nq, H, h, tid);
    const int ty = tid >> 4;   // rows 2ty, 2ty+1
    const int tx = tid & 15;   // blocks tx + 16 jj
    for (int base = 0; base < c; base += kGateChunk) {
      const int nb = min(kGateChunk, c - base);
      for (int i = tid; i < kGateChunk * (D / 4); i += kGateWaves * 64) {
        int j = i / (D / 4), e4 = i % (D / 4);
        f32x4 v = {0.f, 0.f, 0.f, 0.f};
        if (j < nb && gb0 + base + j < total_blocks)
          v = *reinterpret_cast<const f32x4*>(kbar + ((size_t)(gb0 + base + j) * H + h) * D + e4 * 4);
        *reinterpret_cast<f32x4*>(&ks[j][e4 * 4]) = v;
      }
      __syncthreads();
      float acc[2][4];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = 0.f;
#pragma unroll 4
      for (int e = 0; e < D; e += 4) {
        f32x4 qa = *reinterpret_cast<const f32x4*>(&qs[2 * ty][e]);
        f32x4 qb = *reinterpret_cast<const f32x4*>(&qs[2 * ty + 1][e]);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          f32x4 kv = *reinterpret_cast<const f32x4*>(&ks[tx + 16 * jj][e]);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            acc[0][jj] = fmaf(qa[u], kv[u], acc[0][jj]);
            acc[1][jj] = fmaf(qb[u], kv[u], acc[1][jj]);
          }
        }
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        ss[2 * ty][tx + 16 * jj] = acc[0][jj];
        ss[2 * ty + 1][tx + 16 * jj] = acc[1][jj];
      }
      __syncthreads();

#pragma unroll
      for (int i = 0; i < kGateRowsPerWave; ++i) {
        const int r = w * kGateRowsPerWave + i;
        if (r >= nq) continue;  // wave-uniform
        const bool nv = lane < nb;
        const uint32_t nkey = nv ? order_key(ss[r][lane]) : 0u;
        const int32_t nidx = base + lane;
        const bool ov = lane < tcnt[i];
        const uint32_t okey = tkey[i];
        const int32_t oidx = tidx[i];
        const int total = tcnt[i] + nb;
        if (total <= k1) {
          if (ov) { skey[w][lane] = okey; sidx[w][lane] = oidx; }
          if (nv) { skey[w][tcnt[i] + lane] = nkey; sidx[w][tcnt[i] + lane] = nidx; }
          __builtin_amdgcn_wave_barrier();
          tkey[i] = skey[w][lane];
          tidx[i] = sidx[w][lane];
          tcnt[i] = total;
        } else {
          uint32_t prefix = 0u;
          for (int b = 31; b >= 0; --b) {
            const uint32_t cand = prefix | (1u << b);
            const uint64_t mo = __ballot(ov && okey >= cand);
            const uint64_t mn = __ballot(nv && nkey >= cand);
            if (__popcll(mo) + __popcll(mn) >= k1) prefix = cand;
          }
          const uint32_t thr = prefix;
          const uint64_t go = __ballot(ov && okey > thr);
          const uint64_t gn = __ballot(nv && nkey > thr);
          const int need = k1 - __popcll(go) - __popcll(gn);
          const uint64_t eo = __ballot(ov && okey == thr);
          const uint64_t en = __ballot(nv && nkey == thr);
          const int need_n = need - min(need, (int)__popcll(eo));
          const bool selo = ov && (okey > thr || (okey == thr && lanes_below(eo) < need));
          const bool seln = nv && (nkey > thr || (nkey == thr && lanes_below(en) < need_n));
          const uint64_t so = __ballot(selo);
          const uint64_t sn = __ballot(seln);
          __builtin_amdgcn_wave_barrier();
          if (selo) { skey[w][lanes_below(so)] = okey; sidx[w][lanes_below(so)] = oidx; }
          if (seln) {
            const int pos = (int)__popcll(so) + lanes_below(sn);
            skey[w][pos] = nkey;
            sidx[w][pos] = nidx;
          }
          __builtin_amdgcn_wave_barrier();
          tkey[i] = skey[w][lane];
          tidx[i] = sidx[w][lane];
          tcnt[i] = k1;
        }
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

hipError_t launch_gate_topk(const void* q, bool bf16, const float* kbar, const Geo& g,
                            int topk, int32_t* block_idx, hipStream_t st) {
  if (g.total_tokens == 0 || g.max_seqlen == 0) return hipSuccess;
  const int tiles = (g.max_seqlen + kGateRows - 1) / kGateRows;
  dim3 grid(g.num_seqs * tiles, g.num_heads);
  dim3 block(kGateWaves * 64);
#define MOBA_GATE(T, D)                                                                   \
  hipLaunchKernelGGL((gate_topk_kernel<T, D>), grid, block, 0, st, (const T*)q, kbar,     \
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

}  // namespace moba
