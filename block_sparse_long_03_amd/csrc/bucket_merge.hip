// Query bucketing, the transposed-V staging copy and the online-softmax merge.
//
// Bucketing follows "MoBA: Learned Block Sparsity for Long-Context Attention",
// section "Efficiency and Implementation" (queries are arranged according to
// the KV blocks they selected) and step 5 of "MoBA: 面向长上下文大语言模型的
// 混合块注意力机制" (gating-based query-to-block assignment).  The merge is
// the online-softmax combination of the same section: with per-part
// log-sum-exp values lse_p and normalised outputs o_p,
//   lse = ln sum_p exp(lse_p),  o = sum_p exp(lse_p - lse) o_p,
// an exact identity for softmax over the union of the parts' keys.
#include "common.h"
#include "launch.h"

namespace moba {

constexpr int kBucketTokens = 2048;   // tokens per workgroup in count/scatter
constexpr int kBucketLdsBins = 4096;  // LDS histogram limit (past blocks per tile)

// Per (sequence tile, head): histogram of the historical selections in LDS,
// flushed with one global atomic per touched block.
template <bool kScatter>
__global__ __launch_bounds__(256) void bucket_pass_kernel(
    const int32_t* __restrict__ block_idx, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ cu_blocks, int total_tokens, int tiles_per_seq, int H,
    int NB, int block_size, int topk, int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ list) {
  __shared__ int32_t hist[kBucketLdsBins];
  __shared__ int32_t basev[kScatter ? kBucketLdsBins : 1];
  const int sid = blockIdx.x / tiles_per_seq;
  const int tile = blockIdx.x % tiles_per_seq;
  const int h = blockIdx.y;
  int start, len;
  seq_span(cu_seqlens, sid, total_tokens, &start, &len);
  const int p0 = tile * kBucketTokens;
  if (p0 >= len) return;
  const int p1 = min(len, p0 + kBucketTokens);
  const int nbins = (p1 - 1) / block_size;  // past blocks of the last row
  const int gb0 = cu_blocks[sid];
  const bool use_lds = nbins <= kBucketLdsBins;
  int32_t* keyrow = counts + (size_t)h * NB + gb0;

  if (use_lds) {
    for (int b = threadIdx.x; b < nbins; b += 256) hist[b] = 0;
    __syncthreads();
  }
  for (int p = p0 + threadIdx.x; p < p1; p += 256) {
    const int c = p / block_size;
    const int32_t* row = block_idx + ((size_t)(start + p) * H + h) * topk;
    int last = -1, nh = 0;
    for (int j = 0; j < topk; ++j) {
      const int e = row[j];
      if (e >= 0 && e < c && e > last) {
        last = e;
        if (gb0 + e >= NB) { ++nh; continue; }  // inconsistent geometry: drop
        if (!kScatter) {
          if (use_lds) atomicAdd(&hist[e], 1); else atomicAdd(&keyrow[e], 1);
        } else if (!use_lds) {
          const int pos = offsets[(size_t)h * NB + gb0 + e] + atomicAdd(&keyrow[e], 1);
          list[pos] = (start + p) * topk + nh;
        } else {
          atomicAdd(&hist[e], 1);
        }
        ++nh;
      }
    }
  }
  if (!use_lds) return;
  __syncthreads();
  if (!kScatter) {
    for (int b = threadIdx.x; b < nbins; b += 256)
      if (hist[b] && gb0 + b < NB) atomicAdd(&keyrow[b], hist[b]);
    return;
  }
  // scatter: reserve a range per touched block, then place every entry
  for (int b = threadIdx.x; b < nbins; b += 256) {
    const int n = hist[b];
    basev[b] = n && gb0 + b < NB ? offsets[(size_t)h * NB + gb0 + b] + atomicAdd(&keyrow[b], n) : 0;
    hist[b] = 0;
  }
  __syncthreads();
  for (int p = p0 + threadIdx.x; p < p1; p += 256) {
    const int c = p / block_size;
    const int32_t* row = block_idx + ((size_t)(start + p) * H + h) * topk;
    int last = -1, nh = 0;
    for (int j = 0; j < topk; ++j) {
      const int e = row[j];
      if (e >= 0 && e < c && e > last) {
        last = e;
        if (gb0 + e >= NB) { ++nh; continue; }
        list[basev[e] + atomicAdd(&hist[e], 1)] = (start + p) * topk + nh;
        ++nh;
      }
    }
  }
}

// Exclusive scans of the per-(head, block) counts (entries and tiles of
// tile_q rows); clears the counts so the scatter can reuse them as cursors.
__global__ __launch_bounds__(1024) void bucket_scan_kernel(int32_t* __restrict__ counts,
                                                           int n, int tile_q,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ tile_offsets) {
  __shared__ int32_t se[1024];
  __shared__ int32_t stl[1024];
  __shared__ int32_t carry[2];
  if (threadIdx.x == 0) { carry[0] = 0; carry[1] = 0; }
  __syncthreads();
  for (int base = 0; base < n; base += 1024) {
    const int i = base + threadIdx.x;
    const int cval = i < n ? counts[i] : 0;
    const int tval = (cval + tile_q - 1) / tile_q;
    se[threadIdx.x] = cval;
    stl[threadIdx.x] = tval;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      int a = 0, b = 0;
      if (threadIdx.x >= off) { a = se[threadIdx.x - off]; b = stl[threadIdx.x - off]; }
      __syncthreads();
      se[threadIdx.x] += a;
      stl[threadIdx.x] += b;
      __syncthreads();
    }
    if (i < n) {
      offsets[i] = carry[0] + se[threadIdx.x] - cval;
      tile_offsets[i] = carry[1] + stl[threadIdx.x] - tval;
      counts[i] = 0;
    }
    __syncthreads();
    if (threadIdx.x == 1023) { carry[0] += se[1023]; carry[1] += stl[1023]; }
    __syncthreads();
  }
  if (threadIdx.x == 0) { offsets[n] = carry[0]; tile_offsets[n] = carry[1]; }
}

__global__ void fill_zero_kernel(int32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

hipError_t launch_bucket(const int32_t* block_idx, const Geo& g, int topk, int tile_q,
                         int32_t* counts, int32_t* offsets, int32_t* tile_offsets,
                         int32_t* list, hipStream_t st) {
  const int n = g.num_heads * g.total_blocks;
  if (n > 0) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3(min(1024, (n + 255) / 256)), dim3(256), 0, st,
                       counts, n);
  }
  const int tiles = (g.max_seqlen + kBucketTokens - 1) / kBucketTokens;
  dim3 grid(g.num_seqs * tiles, g.num_heads);
  if (tiles > 0 && topk > 1)
    hipLaunchKernelGGL((bucket_pass_kernel<false>), grid, dim3(256), 0, st, block_idx,
                       g.cu_seqlens, g.cu_blocks, g.total_tokens, tiles, g.num_heads,
                       g.total_blocks, g.block_size, topk, counts, offsets, list);
  hipLaunchKernelGGL(bucket_scan_kernel, dim3(1), dim3(1024), 0, st, counts, n, tile_q,
                     offsets, tile_offsets);
  if (tiles > 0 && topk > 1)
    hipLaunchKernelGGL((bucket_pass_kernel<true>), grid, dim3(256), 0, st, block_idx,
                       g.cu_seqlens, g.cu_blocks, g.total_tokens, tiles, g.num_heads,
                       g.total_blocks, g.block_size, topk, counts, offsets, list);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// V^T staging: vt[((gb*H + h)*d + e)*B + p] = V[token of key pi(p), h, e]
// where, inside every group of 16 keys, storage position p holds key
// pi(p) = 8*((p & 7) >> 2) + 4*(p >> 3) + (p & 3) (quads 1 and 2 swapped).
// This is the key order in which a lane of the 32x32x16 MFMA holds its eight
// softmax probabilities, so each lane's eight V^T values are contiguous.
// Keys past the end of the sequence are stored as zero.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void v_transpose_kernel(
    const uint16_t* __restrict__ v, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ cu_blocks, int num_seqs, int total_tokens, int H,
    int block_size, uint16_t* __restrict__ vt) {
  __shared__ uint16_t tile[64][D + 2];
  const int chunks_per_block = block_size / 64;
  const int gb = blockIdx.x / chunks_per_block;
  const int ci = blockIdx.x % chunks_per_block;
  const int h = blockIdx.y;
  const int s = seq_of_block(cu_blocks, num_seqs, gb);
  int start, len;
  seq_span(cu_seqlens, s, total_tokens, &start, &len);
  const int local = (gb - cu_blocks[s]) * block_size + ci * 64;
  const int nk = max(0, min(64, len - local));
  constexpr int SEG = D / 8;
  for (int i = threadIdx.x; i < 64 * SEG; i += 256) {
    const int r = i / SEG, c = i % SEG;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (r < nk) w = *reinterpret_cast<const u32x4*>(v + ((size_t)(start + local + r) * H + h) * D + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[r][c * 8 + 2 * e] = (uint16_t)(w[e] & 0xffffu);
      tile[r][c * 8 + 2 * e + 1] = (uint16_t)(w[e] >> 16);
    }
  }
  __syncthreads();
  uint16_t* dst = vt + ((size_t)gb * H + h) * D * (size_t)block_size + ci * 64;
  for (int i = threadIdx.x; i < D * 8; i += 256) {
    const int e = i / 8, seg = i % 8;  // 8 storage positions per thread
    uint32_t packed[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t two[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int p = seg * 8 + 2 * j + u;
        const int g16 = p & ~15, pp = p & 15;
        const int key = g16 + 8 * ((pp & 7) >> 2) + 4 * (pp >> 3) + (pp & 3);
        two[u] = tile[key][e];
      }
      packed[j] = two[0] | (two[1] << 16);
    }
    u32x4 outv = {packed[0], packed[1], packed[2], packed[3]};
    *reinterpret_cast<u32x4*>(dst + (size_t)e * block_size + seg * 8) = outv;
  }
}

hipError_t launch_v_transpose(const void* v, const Geo& g, uint16_t* vt, hipStream_t st) {
  if (g.total_blocks == 0) return hipSuccess;
  dim3 grid(g.total_blocks * (g.block_size / 64), g.num_heads);
  if (g.head_dim == 128)
    hipLaunchKernelGGL(v_transpose_kernel<128>, grid, dim3(256), 0, st, (const uint16_t*)v,
                       g.cu_seqlens, g.cu_blocks, g.num_seqs, g.total_tokens, g.num_heads,
                       g.block_size, vt);
  else
    hipLaunchKernelGGL(v_transpose_kernel<64>, grid, dim3(256), 0, st, (const uint16_t*)v,
                       g.cu_seqlens, g.cu_blocks, g.num_seqs, g.total_tokens, g.num_heads,
                       g.block_size, vt);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// merge: one wave per (token, head) row
// ---------------------------------------------------------------------------
template <int D, bool kPartBf16, bool kOutBf16>
__global__ __launch_bounds__(256) void merge_kernel(
    const int32_t* __restrict__ block_idx, const int32_t* __restrict__ cu_seqlens,
    int num_seqs, int total_tokens, int H, int block_size, int topk,
    const void* __restrict__ o_part, const float* __restrict__ lse_part,
    void* __restrict__ out, float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (long long)total_tokens * H) return;
  const int t = (int)(row / H);
  const int s = upper_index(cu_seqlens, num_seqs, t);
  const int c = (t - cu_seqlens[s]) / block_size;
  const int32_t* irow = block_idx + row * topk;
  const int nh = count_hist(irow, topk, c);
  const int nparts = nh + 1;
  // part i < nh lives in slot i; the own block in slot topk - 1
  const int my_slot = lane < nh ? lane : topk - 1;
  const float my_lse = lane < nparts ? lse_part[row * topk + my_slot] : -INFINITY;
  const float mx = wave_max(my_lse);
  const float wsum = wave_sum(lane < nparts ? expf(my_lse - mx) : 0.f);
  const float tot = mx + logf(wsum);
  const float my_w = lane < nparts ? expf(my_lse - tot) : 0.f;
  constexpr int PER = D / 64;  // elements per lane
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int i = 0; i < nparts; ++i) {
    const float wi = __shfl(my_w, i);
    const int slot = i < nh ? i : topk - 1;
    const size_t base = ((size_t)row * topk + slot) * D + lane * PER;
    if (kPartBf16) {
      const uint16_t* p = (const uint16_t*)o_part + base;
      if (PER == 2) {
        const uint32_t wv = *reinterpret_cast<const uint32_t*>(p);
        acc[0] = fmaf(wi, lo_bf16(wv), acc[0]);
        acc[PER - 1] = fmaf(wi, hi_bf16(wv), acc[PER - 1]);
      } else {
        acc[0] = fmaf(wi, bf16_bits_to_f32(p[0]), acc[0]);
      }
    } else {
      const float* p = (const float*)o_part + base;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(wi, p[e], acc[e]);
    }
  }
  const size_t ob = (size_t)row * D + lane * PER;
  if (kOutBf16) {
    uint16_t* o = (uint16_t*)out + ob;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = f32_to_bf16_bits(acc[e]);
  } else {
    float* o = (float*)out + ob;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] = acc[e];
  }
  if (lane == 0) lse[row] = tot;
}

hipError_t launch_merge(const int32_t* block_idx, const Geo& g, int topk, const void* o_part,
                        bool part_bf16, const float* lse_part, void* out, bool out_bf16,
                        float* lse, hipStream_t st) {
  const long long rows = (long long)g.total_tokens * g.num_heads;
  if (rows == 0) return hipSuccess;
  dim3 grid((unsigned)((rows + 3) / 4));
#define MOBA_MERGE(D, PB, OB)                                                            \
  hipLaunchKernelGGL((merge_kernel<D, PB, OB>), grid, dim3(256), 0, st, block_idx,       \
                     g.cu_seqlens, g.num_seqs, g.total_tokens, g.num_heads, g.block_size, \
                     topk, o_part, lse_part, out, lse)
  if (g.head_dim == 128) {
    if (part_bf16) { if (out_bf16) MOBA_MERGE(128, true, true); else MOBA_MERGE(128, true, false); }
    else { if (out_bf16) MOBA_MERGE(128, false, true); else MOBA_MERGE(128, false, false); }
  } else {
    if (part_bf16) { if (out_bf16) MOBA_MERGE(64, true, true); else MOBA_MERGE(64, true, false); }
    else { if (out_bf16) MOBA_MERGE(64, false, true); else MOBA_MERGE(64, false, false); }
  }
#undef MOBA_MERGE
  return hipGetLastError();
}

}  // namespace moba
