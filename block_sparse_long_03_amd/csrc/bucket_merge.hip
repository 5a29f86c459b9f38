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
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moba {

constexpr int kBucketTokensMax = 256;  // tokens per workgroup of the count pass (all heads)
constexpr int kBucketLdsBins = 8192;  // LDS histogram limit (heads x past blocks per tile)

// Count pass, per (sequence tile of `tile_tokens` tokens): every (token,
// head) row of block_idx for the HC heads h0 .. h0 + HC - 1 of the group,
// read in memory order (consecutive lanes take consecutive rows, so a wave
// reads one contiguous range per token), counted into an LDS histogram per
// (head of the group, past block) and flushed with one global atomic per
// touched bin.  Dense-prefix rows (dense_row) are skipped; a row below
// dense_blocks that is not one marks its (head, own block) in notfull.
__global__ __launch_bounds__(256) void bucket_count_kernel(
    const int32_t* __restrict__ block_idx, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ cu_blocks, int total_tokens, int tiles_per_seq, int tile_tokens,
    int H, int h0, int HC, int NB, int block_size, int topk, int dense_blocks,
    int32_t* __restrict__ counts, int32_t* __restrict__ notfull) {
  __shared__ int32_t hist[kBucketLdsBins];
  const int sid = blockIdx.x / tiles_per_seq;
  const int tile = blockIdx.x % tiles_per_seq;
  int start, len;
  seq_span(cu_seqlens, sid, total_tokens, &start, &len);
  const int p0 = tile * tile_tokens;
  if (p0 >= len) return;
  const int p1 = min(len, p0 + tile_tokens);
  const int nbins = (p1 - 1) / block_size;  // past blocks of the last row
  const int gb0 = cu_blocks[sid];
  const bool use_lds = nbins * HC <= kBucketLdsBins;
  const int nrows = (p1 - p0) * HC;

  if (use_lds) {
    for (int b = threadIdx.x; b < nbins * HC; b += 256) hist[b] = 0;
    __syncthreads();
  }
  // walks row r = (p - p0) * HC + h of the group (head h0 + h), calling
  // f(h, e) for each accepted historical entry (0 <= e < c, increasing,
  // inside the batch's blocks)
  auto walk = [&](int r, auto&& f) {
    const int p = p0 + r / HC;
    const int h = r - (r / HC) * HC;
    const int c = p / block_size;
    const int32_t* row = block_idx + ((size_t)(start + p) * H + h0 + h) * topk;
    if (c < dense_blocks) {
      if (dense_row(row, topk, c, dense_blocks)) return;
      if (gb0 + c < NB) notfull[(size_t)h * NB + gb0 + c] = 1;
    }
    int last = -1, nh = 0;
    auto visit = [&](int e) {
      if (accept_hist(e, c, last, nh, topk)) {
        last = e;
        if (gb0 + e < NB) f(h, e);  // else inconsistent geometry: dropped
        ++nh;
      }
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
  };
  auto add = [&](int h, int e) {
    if (use_lds) atomicAdd(&hist[h * nbins + e], 1);
    else atomicAdd(&counts[(size_t)h * NB + gb0 + e], 1);
  };
  // kRB rows per thread at a time, all their loads issued before any of them
  // is walked, so that a thread has kRB rows in flight instead of one; the
  // row width KC = topk is a compile-time constant of the walk
  constexpr int kRB = 4;
  auto batched = [&](auto kc_t) {
    constexpr int KC = decltype(kc_t)::value;
    for (int r0 = threadIdx.x; r0 < nrows; r0 += 256 * kRB) {
      int4 e4[kRB][KC / 4];
#pragma unroll
      for (int u = 0; u < kRB; ++u) {
        const int r = min(r0 + 256 * u, nrows - 1);  // rows past the end: loaded, not walked
        const int p = p0 + r / HC, h = r - (r / HC) * HC;
        const int32_t* row = block_idx + ((size_t)(start + p) * H + h0 + h) * KC;
#pragma unroll
        for (int j = 0; j < KC / 4; ++j) e4[u][j] = *reinterpret_cast<const int4*>(row + 4 * j);
      }
#pragma unroll
      for (int u = 0; u < kRB; ++u) {
        const int r = r0 + 256 * u;
        if (r >= nrows) break;
        const int p = p0 + r / HC, h = r - (r / HC) * HC;
        const int c = p / block_size;
        int ev[KC];
#pragma unroll
        for (int j = 0; j < KC / 4; ++j) {
          ev[4 * j] = e4[u][j].x;
          ev[4 * j + 1] = e4[u][j].y;
          ev[4 * j + 2] = e4[u][j].z;
          ev[4 * j + 3] = e4[u][j].w;
        }
        // the accepted historical entries (accept_hist), as walk visits them
        uint32_t accm = 0u;
        int last = -1, nh = 0;
#pragma unroll
        for (int q = 0; q < KC; ++q)
          if (accept_hist(ev[q], c, last, nh, KC)) {
            accm |= 1u << q;
            last = ev[q];
            ++nh;
          }
        if (c < dense_blocks) {
          if (nh == c) continue;  // a dense-prefix row (dense_row)
          if (gb0 + c < NB) notfull[(size_t)h * NB + gb0 + c] = 1;
        }
#pragma unroll
        for (int q = 0; q < KC; ++q)
          if (((accm >> q) & 1u) && gb0 + ev[q] < NB) add(h, ev[q]);
      }
    }
  };
  switch (topk) {
    case 4: batched(std::integral_constant<int, 4>()); break;
    case 8: batched(std::integral_constant<int, 8>()); break;
    case 12: batched(std::integral_constant<int, 12>()); break;
    case 16: batched(std::integral_constant<int, 16>()); break;
    default:
      for (int r = threadIdx.x; r < nrows; r += 256) walk(r, add);
  }
  if (!use_lds) return;
  __syncthreads();
  for (int b = threadIdx.x; b < nbins * HC; b += 256) {
    const int h = b / nbins, e = b - (b / nbins) * nbins;
    if (hist[b]) atomicAdd(&counts[(size_t)h * NB + gb0 + e], hist[b]);
  }
}

// Inclusive sum over the 64 lanes of a wave with DPP adds: row_shr 1, 2, 4, 8
// (zero from outside the 16-lane row) scan each row, then row_bcast:15 adds
// row 0's (row 2's) total to row 1 (row 3) and row_bcast:31 adds the total
// of lanes 0..31 to rows 2 and 3; the rows left out keep 0 (the old value).
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);
  return x;
}

// Scatter of one head's entries of a token tile into the per-(head, block)
// lists, staged in LDS so that every block's run is written by consecutive
// lanes.  The tile's entries are counted per past block into an LDS
// histogram, each non-empty block reserves its range of the list with one
// global atomic, the entries are placed into an LDS staging array grouped by
// block (positions from LDS atomics), and each wave then copies whole runs
// out.  A run of a block holds every entry of the tile's R tokens that
// selected it (about R (k - 1) / n of them), so the list is written in long
// contiguous runs instead of one scattered word per entry.  Tiles whose
// tokens have more past blocks than the LDS histogram holds place their
// entries with global atomics instead.  Workgroups run over (token tile,
// head of the group) with the heads of one tile on one XCD, where they share
// the L2 lines of the tile's block_idx rows.
constexpr int kScatterBins = 1024;
constexpr int kScatterThreads = 1024;  // one token row per thread: the row loads of a walk fly together
constexpr int kScatterStage = 12288;  // staged entries per workgroup

// tokens per scatter tile for rows of k - 1 historical slots: the largest
// power of two in [32, 1024] whose entries fit the staging array
inline int scatter_tile_tokens(int topk) {
  int r = 1024;
  while (r > 32 && (long long)r * (topk - 1) > kScatterStage) r >>= 1;
  return r;
}

__global__ __launch_bounds__(kScatterThreads) void bucket_scatter_kernel(
    const int32_t* __restrict__ block_idx, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ cu_blocks, int total_tokens, int tiles_per_seq, int nunits,
    int tile_tokens, int H, int h0, int HC, int NB, int block_size, int topk, int slot_stride,
    int dense_blocks, const int32_t* __restrict__ notfull, int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ list) {
  __shared__ int32_t hist[kScatterBins];
  __shared__ int32_t loff[kScatterBins + 1];
  __shared__ int32_t gbase[kScatterBins];
  __shared__ int32_t stage[kScatterStage];
  // XCD-contiguous order: workgroup b runs on XCD b % 8; XCD x takes units
  // x, x + 8, ... and, for each, the HC heads one after the other
  const int x = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
  const int unit = x + kXcds * (j / HC);
  const int hl = j % HC;
  if (unit >= nunits) return;
  const int sid = unit / tiles_per_seq;
  const int tile = unit % tiles_per_seq;
  int start, len;
  seq_span(cu_seqlens, sid, total_tokens, &start, &len);
  const int p0 = tile * tile_tokens;
  if (p0 >= len) return;
  const int p1 = min(len, p0 + tile_tokens);
  const int nbins = (p1 - 1) / block_size;  // past blocks of the last row
  if (nbins == 0) return;
  const int gb0 = cu_blocks[sid];
  const size_t key0 = (size_t)hl * NB + gb0;
  // a block below dense_blocks whose notfull flag is 0 holds only
  // dense-prefix rows: they are skipped without reading them, and a tile of
  // such blocks has nothing to do
  auto all_dense = [&](int cb) {
    return cb < dense_blocks && gb0 + cb < NB && notfull[key0 + cb] == 0;
  };
  {
    bool skip = true;
    for (int cb = p0 / block_size; cb <= (p1 - 1) / block_size && skip; ++cb)
      skip = all_dense(cb);
    if (skip) return;
  }
  // calls f(e, slot, p) for each accepted historical entry of row p (the
  // rule of accept_hist, inside the batch's blocks): at most topk - 1 per
  // row, so a tile stages at most tile_tokens * (topk - 1) entries
  auto walk = [&](int p, auto&& f) {
    const int c = p / block_size;
    if (all_dense(c)) return;
    const int32_t* row = block_idx + ((size_t)(start + p) * H + h0 + hl) * topk;
    if (dense_row(row, topk, c, dense_blocks)) return;
    int last = -1, nh = 0;
    auto visit = [&](int e) {
      if (accept_hist(e, c, last, nh, topk)) {
        last = e;
        if (gb0 + e < NB) f(e, nh, p);  // else inconsistent geometry: dropped
        ++nh;
      }
    };
    if ((topk & 3) == 0) {
      for (int q = 0; q < topk; q += 4) {
        const int4 e4 = *reinterpret_cast<const int4*>(row + q);
        visit(e4.x);
        visit(e4.y);
        visit(e4.z);
        visit(e4.w);
      }
    } else {
      for (int q = 0; q < topk; ++q) visit(row[q]);
    }
  };
  auto value = [&](int slot, int p) {
    return slot_stride ? (start + p) * slot_stride + slot : start + p;
  };
  if (nbins > kScatterBins) {
    for (int p = p0 + (int)threadIdx.x; p < p1; p += kScatterThreads)
      walk(p, [&](int e, int slot, int pp) {
        const size_t key = key0 + e;
        list[offsets[key] + atomicAdd(&counts[key], 1)] = value(slot, pp);
      });
    return;
  }
  for (int b = threadIdx.x; b < nbins; b += kScatterThreads) hist[b] = 0;
  __syncthreads();
  // k <= kCacheK: the thread's one row (tiles hold at most kScatterThreads
  // tokens) is read once, its entries kept in registers with the mask of
  // accepted ones for the staging pass
  constexpr int kCacheK = 16;
  const bool cached = topk <= kCacheK;
  const int p_me = p0 + (int)threadIdx.x;
  int ev[kCacheK];
  uint32_t accm = 0u;
  if (cached) {
    if (p_me < p1) {
      const int c = p_me / block_size;
      if (!all_dense(c)) {
        const int32_t* row = block_idx + ((size_t)(start + p_me) * H + h0 + hl) * topk;
        if ((topk & 3) == 0) {
#pragma unroll
          for (int q = 0; q < kCacheK; q += 4) {
            int4 e4 = {-1, -1, -1, -1};
            if (q < topk) e4 = *reinterpret_cast<const int4*>(row + q);
            ev[q] = e4.x; ev[q + 1] = e4.y; ev[q + 2] = e4.z; ev[q + 3] = e4.w;
          }
        } else {
#pragma unroll
          for (int q = 0; q < kCacheK; ++q) ev[q] = q < topk ? row[q] : -1;
        }
        int last = -1, nh = 0;
#pragma unroll
        for (int q = 0; q < kCacheK; ++q)
          if (q < topk && accept_hist(ev[q], c, last, nh, topk)) {
            accm |= 1u << q;
            last = ev[q];
            ++nh;
          }
        if (c < dense_blocks && nh == c) accm = 0u;  // a dense-prefix row
#pragma unroll
        for (int q = 0; q < kCacheK; ++q)
          if (((accm >> q) & 1u) && gb0 + ev[q] < NB) atomicAdd(&hist[ev[q]], 1);
      }
    }
  } else {
    for (int p = p0 + (int)threadIdx.x; p < p1; p += kScatterThreads)
      walk(p, [&](int e, int, int) { atomicAdd(&hist[e], 1); });
  }
  __syncthreads();
  // exclusive scan of the histogram (one wave), global range per block
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    int carry = 0;
    for (int b0 = 0; b0 < nbins; b0 += 64) {
      const int b = b0 + lane;
      const int v = b < nbins ? hist[b] : 0;
      const int inc = wave_incl_scan(v);
      if (b < nbins) loff[b] = carry + inc - v;
      carry += __builtin_amdgcn_readlane(inc, 63);
    }
    if (lane == 0) loff[nbins] = carry;
  }
  __syncthreads();
  // each block's range of the list (one bin per thread: nbins <= kScatterBins
  // <= kScatterThreads): the reservation is issued here and its result used
  // only after the staging, behind a barrier that waits for LDS alone, so
  // the atomic's round trip overlaps the staging
  static_assert(kScatterBins <= kScatterThreads, "one bin per thread");
  const int bme = threadIdx.x;
  int n_me = 0, off_me = 0, res_me = 0;
  if (bme < nbins) {
    n_me = hist[bme];
    hist[bme] = 0;
    if (n_me) {
      off_me = offsets[key0 + bme];
      res_me = atomicAdd(&counts[key0 + bme], n_me);
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (cached) {
#pragma unroll
    for (int q = 0; q < kCacheK; ++q)
      if (((accm >> q) & 1u) && gb0 + ev[q] < NB)
        stage[loff[ev[q]] + atomicAdd(&hist[ev[q]], 1)] =
            value(__popc(accm & ((1u << q) - 1u)), p_me);
  } else {
    for (int p = p0 + (int)threadIdx.x; p < p1; p += kScatterThreads)
      walk(p, [&](int e, int slot, int pp) {
        stage[loff[e] + atomicAdd(&hist[e], 1)] = value(slot, pp);
      });
  }
  if (bme < nbins) gbase[bme] = n_me ? off_me + res_me : 0;
  __syncthreads();
  // each wave copies whole runs: lanes write consecutive list entries
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int b = wv; b < nbins; b += kScatterThreads / 64) {
    const int a = loff[b], n = loff[b + 1] - a;
    int32_t* dst = list + gbase[b];
    for (int i = lane; i < n; i += 64) dst[i] = stage[a + i];
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

__global__ __launch_bounds__(256) void tile_info_kernel(const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ tile_offsets,
                                                        int nkeys, int tile_q, long long max_tiles,
                                                        int4* __restrict__ info) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= max_tiles) return;
  const int total = tile_offsets[nkeys];
  if (t >= total) {
    info[t] = make_int4(-1, 0, 0, 0);
    return;
  }
  const int key = upper_index(tile_offsets, nkeys, (int)t);
  const int e0 = offsets[key] + ((int)t - tile_offsets[key]) * tile_q;
  const int e1 = min(offsets[key + 1], e0 + tile_q);
  info[t] = make_int4(key, e0, e1, 0);
}

__global__ void fill_zero_kernel(int32_t* __restrict__ p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

hipError_t launch_bucket(const int32_t* block_idx, const Geo& g, int topk, int tile_q,
                         int32_t* counts, int32_t* offsets, int32_t* tile_offsets,
                         int32_t* list, int4* tile_info, long long max_tiles, hipStream_t st,
                         bool tokens_only, int dense_blocks, int32_t* notfull) {
  const int slot_stride = tokens_only ? 0 : topk;
  const int n = g.head_cnt * g.total_blocks;
  if (n > 0) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3(min(1024, (n + 255) / 256)), dim3(256), 0, st,
                       counts, n);
    if (dense_blocks > 0)
      hipLaunchKernelGGL(fill_zero_kernel, dim3(min(1024, (n + 255) / 256)), dim3(256), 0, st,
                         notfull, n);
  }
  // tiles of 32..256 tokens, small enough for about 1024 workgroups
  int tile_tokens = kBucketTokensMax;
  while (tile_tokens > 32 && (long long)g.total_tokens < 1024LL * tile_tokens) tile_tokens >>= 1;
  const int tiles = (g.max_seqlen + tile_tokens - 1) / tile_tokens;
  dim3 grid(g.num_seqs * tiles);
  if (tiles > 0 && topk > 1)
    hipLaunchKernelGGL(bucket_count_kernel, grid, dim3(256), 0, st, block_idx, g.cu_seqlens,
                       g.cu_blocks, g.total_tokens, tiles, tile_tokens, g.num_heads, g.head_lo,
                       g.head_cnt, g.total_blocks, g.block_size, topk, dense_blocks, counts,
                       notfull);
  hipLaunchKernelGGL(bucket_scan_kernel, dim3(1), dim3(1024), 0, st, counts, n, tile_q,
                     offsets, tile_offsets);
  if (tiles > 0 && topk > 1) {
    const int rt = scatter_tile_tokens(topk);
    const int stiles = (g.max_seqlen + rt - 1) / rt;
    const int nunits = g.num_seqs * stiles;
    const long long wgs = (long long)((nunits + kXcds - 1) / kXcds) * kXcds * g.head_cnt;
    hipLaunchKernelGGL(bucket_scatter_kernel, dim3((unsigned)wgs), dim3(kScatterThreads), 0, st,
                       block_idx,
                       g.cu_seqlens, g.cu_blocks, g.total_tokens, stiles, nunits, rt,
                       g.num_heads, g.head_lo, g.head_cnt, g.total_blocks, g.block_size, topk,
                       slot_stride, dense_blocks, notfull, counts, offsets, list);
  }
  if (tile_info && max_tiles > 0)
    hipLaunchKernelGGL(tile_info_kernel, dim3((unsigned)((max_tiles + 255) / 256)), dim3(256), 0,
                       st, offsets, tile_offsets, n, tile_q, max_tiles, tile_info);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// V staging for the MFMA kernels, in two passes:
//  1. vmax_bits[h] = fp32 bits of max |v| over head h (atomicMax on the bit
//     patterns, which order like the values for non-negative floats);
//  2. vt[((gb*H + h)*d + e)*B + p] = fp16(V[token of key pi(p), h, e] * 2^-e_h)
//     with e_h = v_exponent(vmax_bits[h]) (exact for bf16 input), where,
//     inside every group of 16 keys, storage position p holds key
//     pi(p) = 8*((p & 7) >> 2) + 4*(p >> 3) + (p & 3) (quads 1 and 2
//     swapped): the key order in which a lane of the 32x32x16 MFMA holds its
//     eight softmax probabilities, so each lane's eight V^T values are one
//     16-byte read.  Keys past the end of the sequence are stored as zero.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void vmax_kernel(const uint16_t* __restrict__ v,
                                                   int total_tokens, int hd, int head_dim,
                                                   int h0, int span,
                                                   uint32_t* __restrict__ vmax_bits) {
  __shared__ uint32_t red[256];
  const int col0 = h0 * head_dim + blockIdx.y * 64;  // 64 columns of one head
  const int tx = threadIdx.x & 7, ty = threadIdx.x >> 3;
  const long long t0 = (long long)blockIdx.x * span;  // span tokens per workgroup
  uint32_t m = 0u;
  const int t_end = (int)min((long long)total_tokens, t0 + span);
  for (int t = (int)t0 + ty; t < t_end; t += 32) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(v + (size_t)t * hd + col0 + tx * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m = max(m, (w[i] << 16) & 0x7fffffffu);
      m = max(m, w[i] & 0x7fff0000u);
    }
  }
  red[threadIdx.x] = m;
  __syncthreads();
  for (int st = 128; st >= 1; st >>= 1) {
    if (threadIdx.x < st) red[threadIdx.x] = max(red[threadIdx.x], red[threadIdx.x + st]);
    __syncthreads();
  }
  if (threadIdx.x == 0) atomicMax(&vmax_bits[col0 / head_dim - h0], red[0]);
}

template <int D>
__global__ __launch_bounds__(256) void v_transpose_kernel(
    const uint16_t* __restrict__ v, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ cu_blocks, int num_seqs, int total_tokens, int H, int h0,
    int block_size, const uint32_t* __restrict__ vmax_bits, uint16_t* __restrict__ vt) {
  __shared__ float tile[64][D + 1];
  const int HC = gridDim.y;  // heads of the group; h below is the place in it
  const int chunks_per_block = block_size / 64;
  const int gb = blockIdx.x / chunks_per_block;
  const int ci = blockIdx.x % chunks_per_block;
  const int h = blockIdx.y;
  const int s = seq_of_block(cu_blocks, num_seqs, gb);
  int start, len;
  seq_span(cu_seqlens, s, total_tokens, &start, &len);
  const int local = (gb - cu_blocks[s]) * block_size + ci * 64;
  const int nk = max(0, min(64, len - local));
  const float scale = __builtin_ldexpf(1.0f, -v_exponent(vmax_bits[h]));
  constexpr int SEG = D / 8;
  for (int i = threadIdx.x; i < 64 * SEG; i += 256) {
    const int r = i / SEG, c = i % SEG;
    u32x4 w = {0u, 0u, 0u, 0u};
    if (r < nk)
      w = *reinterpret_cast<const u32x4*>(v + ((size_t)(start + local + r) * H + h0 + h) * D + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[r][c * 8 + 2 * e] = lo_bf16(w[e]) * scale;
      tile[r][c * 8 + 2 * e + 1] = hi_bf16(w[e]) * scale;
    }
  }
  __syncthreads();
  uint16_t* dst = vt + ((size_t)gb * HC + h) * D * (size_t)block_size + ci * 64;
  for (int i = threadIdx.x; i < D * 8; i += 256) {
    const int e = i / 8, seg = i % 8;  // 8 storage positions per thread
    uint32_t packed[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float two[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int p = seg * 8 + 2 * j + u;
        const int g16 = p & ~15, pp = p & 15;
        const int key = g16 + 8 * ((pp & 7) >> 2) + 4 * (pp >> 3) + (pp & 3);
        two[u] = tile[key][e];
      }
      packed[j] = pack_f16x2(two[0], two[1]);
    }
    u32x4 outv = {packed[0], packed[1], packed[2], packed[3]};
    *reinterpret_cast<u32x4*>(dst + (size_t)e * block_size + seg * 8) = outv;
  }
}

hipError_t launch_v_transpose(const void* v, const Geo& g, uint32_t* vmax_bits, uint16_t* vt,
                              hipStream_t st) {
  if (g.total_blocks == 0) return hipSuccess;
  const int hd = g.num_heads * g.head_dim;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(1), dim3(256), 0, st, (int32_t*)vmax_bits,
                     g.head_cnt);
  // 2048 tokens per workgroup, fewer (down to 256) while that leaves the
  // grid under 2048 workgroups
  const int cols = g.head_cnt * g.head_dim / 64;
  int span = 2048;
  while (span > 256 && (long long)((g.total_tokens + span - 1) / span) * cols < 2048) span /= 2;
  hipLaunchKernelGGL(vmax_kernel, dim3((g.total_tokens + span - 1) / span, cols), dim3(256), 0,
                     st, (const uint16_t*)v, g.total_tokens, hd, g.head_dim, g.head_lo, span,
                     vmax_bits);
  dim3 grid(g.total_blocks * (g.block_size / 64), g.head_cnt);
  if (g.head_dim == 128)
    hipLaunchKernelGGL(v_transpose_kernel<128>, grid, dim3(256), 0, st, (const uint16_t*)v,
                       g.cu_seqlens, g.cu_blocks, g.num_seqs, g.total_tokens, g.num_heads,
                       g.head_lo, g.block_size, vmax_bits, vt);
  else
    hipLaunchKernelGGL(v_transpose_kernel<64>, grid, dim3(256), 0, st, (const uint16_t*)v,
                       g.cu_seqlens, g.cu_blocks, g.num_seqs, g.total_tokens, g.num_heads,
                       g.head_lo, g.block_size, vmax_bits, vt);
  return hipGetLastError();
}

// Butterfly steps across the 16 lanes of a merge row as DPP moves (VALU, no
// LDS round trip): lane ^ 8 is row_ror:8 (a 16-lane row rotated by half),
// lane ^ 4 quad_perm [3,2,1,0] (lane ^ 3) then row_half_mirror (lane ^ 7),
// lane ^ 2 and lane ^ 1 one quad_perm each.
__device__ __forceinline__ float row16_xor(float v, int m) {
  const int x = __float_as_int(v);
  if (m == 8) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false));
  if (m == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));
  if (m == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));
  const int y = __builtin_amdgcn_mov_dpp(x, 0x1B, 0xF, 0xF, false);
  return __int_as_float(__builtin_amdgcn_mov_dpp(y, 0x141, 0xF, 0xF, false));
}

// ---------------------------------------------------------------------------
// merge: 16 lanes per (token, head) row, 16 rows per workgroup.  Each lane
// owns D/16 consecutive output dims; the part weights exp(lse_p - lse) go
// through LDS so that every lane can stream its slice of all the parts with
// several loads in flight.  The fp16 partials are read once, with
// non-temporal loads (5-7% faster than plain ones).  Rows are those of the HC heads h0 .. h0 + HC - 1:
// partials and V scales are indexed by the head's place in that group,
// block_idx, out and lse by its global head.
// ---------------------------------------------------------------------------
template <int D, bool kPartF16, bool kOutBf16>
__global__ __launch_bounds__(256) void merge_kernel(
    const int32_t* __restrict__ block_idx, const int32_t* __restrict__ cu_seqlens,
    int num_seqs, int total_tokens, int H, int h0, int HC, int block_size, int topk,
    int dense_blocks, const void* __restrict__ o_part, const float* __restrict__ lse_part,
    const uint32_t* __restrict__ vmax_bits, void* __restrict__ out, float* __restrict__ lse) {
  constexpr int PER = D / 16;  // output dims per lane
  __shared__ float wts[16][64];
  __shared__ int slots[16][64];
  const int r16 = threadIdx.x >> 4;  // row within the workgroup
  const int li = threadIdx.x & 15;   // lane within the row
  const long long row = (long long)blockIdx.x * 16 + r16;  // (token, head of the group)
  const bool valid = row < (long long)total_tokens * HC;
  const int t = (int)(row / HC);
  const int hl = (int)(row - (long long)t * HC);
  const long long grow = (long long)t * H + h0 + hl;       // (token, global head)
  int nparts = 0;
  float tot = 0.f;
  bool dense = false;  // written by the dense-prefix pass
  if (valid) {
    const int s = upper_index(cu_seqlens, num_seqs, t);
    const int c = (t - cu_seqlens[s]) / block_size;
    const int nh = count_hist(block_idx + grow * topk, topk, c);
    dense = c < dense_blocks && nh == c;
    nparts = dense ? 0 : nh + 1;  // dense-prefix rows: no partials to weigh
    // part i < nh lives in slot i; the own block in slot topk - 1
    float l4[4];
    float mx = -INFINITY;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = li + 16 * u;
      const int slot = i < nh ? i : topk - 1;
      l4[u] = i < nparts ? lse_part[row * topk + slot] : -INFINITY;
      mx = fmaxf(mx, l4[u]);
      if (i < 64) slots[r16][i] = slot;
    }
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) mx = fmaxf(mx, row16_xor(mx, o));
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) sum += (li + 16 * u < nparts) ? expf(l4[u] - mx) : 0.f;
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) sum += row16_xor(sum, o);
    tot = mx + logf(sum);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = li + 16 * u;
      if (i < 64) wts[r16][i] = i < nparts ? expf(l4[u] - tot) : 0.f;
    }
  }
  __syncthreads();
  if (!valid || dense) return;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  const size_t rbase = (size_t)row * topk;
  int i = 0;
  for (; i + 4 <= nparts; i += 4) {
    float v[4][PER];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const size_t base = (rbase + slots[r16][i + u]) * D + li * PER;
      if (kPartF16) {
        const uint16_t* p = (const uint16_t*)o_part + base;
        if (PER == 8) {
          const u32x4 w4 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
          for (int e = 0; e < 4; ++e) { v[u][2 * e] = lo_f16(w4[e]); v[u][2 * e + 1] = hi_f16(w4[e]); }
        } else {
          const u32x2 w2 = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
#pragma unroll
          for (int e = 0; e < 2; ++e) { v[u][2 * e] = lo_f16(w2[e]); v[u][2 * e + 1] = hi_f16(w2[e]); }
        }
      } else {
        const float* p = (const float*)o_part + base;
#pragma unroll
        for (int e = 0; e < PER; e += 4) {
          const f32x4 f4 = *reinterpret_cast<const f32x4*>(p + e);
#pragma unroll
          for (int z = 0; z < 4; ++z) v[u][e + z] = f4[z];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float wi = wts[r16][i + u];
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(wi, v[u][e], acc[e]);
    }
  }
  for (; i < nparts; ++i) {
    const size_t base = (rbase + slots[r16][i]) * D + li * PER;
    const float wi = wts[r16][i];
    if (kPartF16) {
      const uint16_t* p = (const uint16_t*)o_part + base;
#pragma unroll
      for (int e = 0; e < PER; e += 2) {
        const uint32_t w2 = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p + e));
        acc[e] = fmaf(wi, lo_f16(w2), acc[e]);
        acc[e + 1] = fmaf(wi, hi_f16(w2), acc[e + 1]);
      }
    } else {
      const float* p = (const float*)o_part + base;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(wi, p[e], acc[e]);
    }
  }
  if (kPartF16) {
    // fp16 partials are in units of 2^-e_h (the staged V's scale)
    const float sc = __builtin_ldexpf(1.0f, v_exponent(vmax_bits[hl]));
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] *= sc;
  }
  const size_t ob = (size_t)grow * D + li * PER;
  if (kOutBf16) {
    uint32_t* o = (uint32_t*)((uint16_t*)out + ob);
#pragma unroll
    for (int e = 0; e < PER; e += 2) o[e / 2] = pack_bf16x2(acc[e], acc[e + 1]);
  } else {
    float* o = (float*)out + ob;
#pragma unroll
    for (int e = 0; e < PER; e += 4) {
      f32x4 f4 = {acc[e], acc[e + 1], acc[e + 2], acc[e + 3]};
      *reinterpret_cast<f32x4*>(o + e) = f4;
    }
  }
  if (li == 0) lse[grow] = tot;
}

hipError_t launch_merge(const int32_t* block_idx, const Geo& g, int topk, int dense_blocks,
                        const void* o_part, bool part_f16, const float* lse_part,
                        const uint32_t* vmax_bits, void* out, bool out_bf16, float* lse,
                        hipStream_t st) {
  const long long rows = (long long)g.total_tokens * g.head_cnt;
  if (rows == 0) return hipSuccess;
  dim3 grid((unsigned)((rows + 15) / 16));
#define MOBA_MERGE(D, PB, OB)                                                            \
  hipLaunchKernelGGL((merge_kernel<D, PB, OB>), grid, dim3(256), 0, st, block_idx,       \
                     g.cu_seqlens, g.num_seqs, g.total_tokens, g.num_heads, g.head_lo,    \
                     g.head_cnt, g.block_size, topk, dense_blocks, o_part, lse_part, vmax_bits, \
                     out, lse)
  if (g.head_dim == 128) {
    if (part_f16) { if (out_bf16) MOBA_MERGE(128, true, true); else MOBA_MERGE(128, true, false); }
    else { if (out_bf16) MOBA_MERGE(128, false, true); else MOBA_MERGE(128, false, false); }
  } else {
    if (part_f16) { if (out_bf16) MOBA_MERGE(64, true, true); else MOBA_MERGE(64, true, false); }
    else { if (out_bf16) MOBA_MERGE(64, false, true); else MOBA_MERGE(64, false, false); }
  }
#undef MOBA_MERGE
  return hipGetLastError();
}

}  // namespace moba
