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

constexpr int kBucketTokensMax = 256;  // tokens per workgroup in count/scatter (all heads)
constexpr int kBucketLdsBins = 8192;  // LDS histogram limit (heads x past blocks per tile)

// Per (sequence tile of `tile_tokens` tokens): every (token, head) row of
// block_idx, read in memory order (consecutive lanes take consecutive rows,
// so a wave reads one contiguous range), counted into an LDS histogram per
// (head, past block) and flushed with one global atomic per touched bin.
// The scatter pass reserves a range per bin, then places each entry: the
// global token times slot_stride plus its slot, or (slot_stride 0) the token
// alone.
template <bool kScatter>
__global__ __launch_bounds__(256) void bucket_pass_kernel(
    const int32_t* __restrict__ block_idx, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ cu_blocks, int total_tokens, int tiles_per_seq, int tile_tokens,
    int H, int NB, int block_size, int topk, int slot_stride, int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ list) {
  __shared__ int32_t hist[kBucketLdsBins];
  __shared__ int32_t basev[kScatter ? kBucketLdsBins : 1];
  const int sid = blockIdx.x / tiles_per_seq;
  const int tile = blockIdx.x % tiles_per_seq;
  int start, len;
  seq_span(cu_seqlens, sid, total_tokens, &start, &len);
  const int p0 = tile * tile_tokens;
  if (p0 >= len) return;
  const int p1 = min(len, p0 + tile_tokens);
  const int nbins = (p1 - 1) / block_size;  // past blocks of the last row
  const int gb0 = cu_blocks[sid];
  const bool use_lds = nbins * H <= kBucketLdsBins;
  const int nrows = (p1 - p0) * H;
  const int32_t* rows = block_idx + ((size_t)(start + p0) * H) * topk;

  if (use_lds) {
    for (int b = threadIdx.x; b < nbins * H; b += 256) hist[b] = 0;
    __syncthreads();
  }
  // walks row r = (p - p0) * H + h, calling f(h, e, slot) for each accepted
  // historical entry (0 <= e < c, increasing, inside the batch's blocks)
  auto walk = [&](int r, auto&& f) {
    const int p = p0 + r / H;
    const int h = r - (r / H) * H;
    const int c = p / block_size;
    const int32_t* row = rows + (size_t)r * topk;
    int last = -1, nh = 0;
    auto visit = [&](int e) {
      if (e >= 0 && e < c && e > last) {
        last = e;
        if (gb0 + e < NB) f(h, e, nh, p);  // else inconsistent geometry: dropped
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
  if (!kScatter) {
    for (int r = threadIdx.x; r < nrows; r += 256)
      walk(r, [&](int h, int e, int, int) {
        if (use_lds) atomicAdd(&hist[h * nbins + e], 1);
        else atomicAdd(&counts[(size_t)h * NB + gb0 + e], 1);
      });
    if (!use_lds) return;
    __syncthreads();
    for (int b = threadIdx.x; b < nbins * H; b += 256) {
      const int h = b / nbins, e = b - (b / nbins) * nbins;
      if (hist[b]) atomicAdd(&counts[(size_t)h * NB + gb0 + e], hist[b]);
    }
    return;
  }
  if (!use_lds) {
    for (int r = threadIdx.x; r < nrows; r += 256)
      walk(r, [&](int h, int e, int slot, int p) {
        const size_t key = (size_t)h * NB + gb0 + e;
        list[offsets[key] + atomicAdd(&counts[key], 1)] = slot_stride ? (start + p) * slot_stride + slot : start + p;
      });
    return;
  }
  for (int r = threadIdx.x; r < nrows; r += 256)
    walk(r, [&](int h, int e, int, int) { atomicAdd(&hist[h * nbins + e], 1); });
  __syncthreads();
  // reserve a range per touched bin, then place every entry
  for (int b = threadIdx.x; b < nbins * H; b += 256) {
    const int h = b / nbins, e = b - (b / nbins) * nbins;
    const int n = hist[b];
    const size_t key = (size_t)h * NB + gb0 + e;
    basev[b] = n ? offsets[key] + atomicAdd(&counts[key], n) : 0;
    hist[b] = 0;
  }
  __syncthreads();
  for (int r = threadIdx.x; r < nrows; r += 256)
    walk(r, [&](int h, int e, int slot, int p) {
      const int b = h * nbins + e;
      list[basev[b] + atomicAdd(&hist[b], 1)] = slot_stride ? (start + p) * slot_stride + slot : start + p;
    });
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
                         bool tokens_only) {
  const int slot_stride = tokens_only ? 0 : topk;
  const int n = g.num_heads * g.total_blocks;
  if (n > 0) {
    hipLaunchKernelGGL(fill_zero_kernel, dim3(min(1024, (n + 255) / 256)), dim3(256), 0, st,
                       counts, n);
  }
  // tiles of 32..256 tokens, small enough for about 1024 workgroups
  int tile_tokens = kBucketTokensMax;
  while (tile_tokens > 32 && (long long)g.total_tokens < 1024LL * tile_tokens) tile_tokens >>= 1;
  const int tiles = (g.max_seqlen + tile_tokens - 1) / tile_tokens;
  dim3 grid(g.num_seqs * tiles);
  if (tiles > 0 && topk > 1)
    hipLaunchKernelGGL((bucket_pass_kernel<false>), grid, dim3(256), 0, st, block_idx,
                       g.cu_seqlens, g.cu_blocks, g.total_tokens, tiles, tile_tokens, g.num_heads,
                       g.total_blocks, g.block_size, topk, slot_stride, counts, offsets, list);
  hipLaunchKernelGGL(bucket_scan_kernel, dim3(1), dim3(1024), 0, st, counts, n, tile_q,
                     offsets, tile_offsets);
  if (tiles > 0 && topk > 1)
    hipLaunchKernelGGL((bucket_pass_kernel<true>), grid, dim3(256), 0, st, block_idx,
                       g.cu_seqlens, g.cu_blocks, g.total_tokens, tiles, tile_tokens, g.num_heads,
                       g.total_blocks, g.block_size, topk, slot_stride, counts, offsets, list);
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
                                                   uint32_t* __restrict__ vmax_bits) {
  __shared__ uint32_t red[256];
  const int col0 = blockIdx.y * 64;          // 64 columns of one head
  const int tx = threadIdx.x & 7, ty = threadIdx.x >> 3;
  const int t0 = blockIdx.x * 2048;
  uint32_t m = 0u;
  for (int t = t0 + ty; t < min(total_tokens, t0 + 2048); t += 32) {
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
  if (threadIdx.x == 0) atomicMax(&vmax_bits[col0 / head_dim], red[0]);
}

template <int D>
__global__ __launch_bounds__(256) void v_transpose_kernel(
    const uint16_t* __restrict__ v, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ cu_blocks, int num_seqs, int total_tokens, int H,
    int block_size, const uint32_t* __restrict__ vmax_bits, uint16_t* __restrict__ vt) {
  __shared__ float tile[64][D + 1];
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
    if (r < nk) w = *reinterpret_cast<const u32x4*>(v + ((size_t)(start + local + r) * H + h) * D + c * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[r][c * 8 + 2 * e] = lo_bf16(w[e]) * scale;
      tile[r][c * 8 + 2 * e + 1] = hi_bf16(w[e]) * scale;
    }
  }
  __syncthreads();
  uint16_t* dst = vt + ((size_t)gb * H + h) * D * (size_t)block_size + ci * 64;
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
                     g.num_heads);
  hipLaunchKernelGGL(vmax_kernel, dim3((g.total_tokens + 2047) / 2048, hd / 64), dim3(256), 0, st,
                     (const uint16_t*)v, g.total_tokens, hd, g.head_dim, vmax_bits);
  dim3 grid(g.total_blocks * (g.block_size / 64), g.num_heads);
  if (g.head_dim == 128)
    hipLaunchKernelGGL(v_transpose_kernel<128>, grid, dim3(256), 0, st, (const uint16_t*)v,
                       g.cu_seqlens, g.cu_blocks, g.num_seqs, g.total_tokens, g.num_heads,
                       g.block_size, vmax_bits, vt);
  else
    hipLaunchKernelGGL(v_transpose_kernel<64>, grid, dim3(256), 0, st, (const uint16_t*)v,
                       g.cu_seqlens, g.cu_blocks, g.num_seqs, g.total_tokens, g.num_heads,
                       g.block_size, vmax_bits, vt);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// merge: 16 lanes per (token, head) row, 16 rows per workgroup.  Each lane
// owns D/16 consecutive output dims; the part weights exp(lse_p - lse) go
// through LDS so that every lane can stream its slice of all the parts with
// several loads in flight.
// ---------------------------------------------------------------------------
template <int D, bool kPartF16, bool kOutBf16>
__global__ __launch_bounds__(256) void merge_kernel(
    const int32_t* __restrict__ block_idx, const int32_t* __restrict__ cu_seqlens,
    int num_seqs, int total_tokens, int H, int block_size, int topk,
    const void* __restrict__ o_part, const float* __restrict__ lse_part,
    const uint32_t* __restrict__ vmax_bits, void* __restrict__ out, float* __restrict__ lse) {
  constexpr int PER = D / 16;  // output dims per lane
  __shared__ float wts[16][64];
  __shared__ int slots[16][64];
  const int r16 = threadIdx.x >> 4;  // row within the workgroup
  const int li = threadIdx.x & 15;   // lane within the row
  const long long row = (long long)blockIdx.x * 16 + r16;
  const bool valid = row < (long long)total_tokens * H;
  int nparts = 0;
  float tot = 0.f;
  if (valid) {
    const int t = (int)(row / H);
    const int s = upper_index(cu_seqlens, num_seqs, t);
    const int c = (t - cu_seqlens[s]) / block_size;
    const int nh = count_hist(block_idx + row * topk, topk, c);
    nparts = nh + 1;
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
    for (int o = 8; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o, 16));
    float sum = 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u) sum += (li + 16 * u < nparts) ? expf(l4[u] - mx) : 0.f;
    for (int o = 8; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 16);
    tot = mx + logf(sum);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = li + 16 * u;
      if (i < 64) wts[r16][i] = i < nparts ? expf(l4[u] - tot) : 0.f;
    }
  }
  __syncthreads();
  if (!valid) return;
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
          const u32x4 w4 = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
          for (int e = 0; e < 4; ++e) { v[u][2 * e] = lo_f16(w4[e]); v[u][2 * e + 1] = hi_f16(w4[e]); }
        } else {
          const u32x2 w2 = *reinterpret_cast<const u32x2*>(p);
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
        const uint32_t w2 = *reinterpret_cast<const uint32_t*>(p + e);
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
    const float sc = __builtin_ldexpf(1.0f, v_exponent(vmax_bits[row % H]));
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] *= sc;
  }
  const size_t ob = (size_t)row * D + li * PER;
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
  if (li == 0) lse[row] = tot;
}

hipError_t launch_merge(const int32_t* block_idx, const Geo& g, int topk, const void* o_part,
                        bool part_f16, const float* lse_part, const uint32_t* vmax_bits,
                        void* out, bool out_bf16, float* lse, hipStream_t st) {
  const long long rows = (long long)g.total_tokens * g.num_heads;
  if (rows == 0) return hipSuccess;
  dim3 grid((unsigned)((rows + 15) / 16));
#define MOBA_MERGE(D, PB, OB)                                                            \
  hipLaunchKernelGGL((merge_kernel<D, PB, OB>), grid, dim3(256), 0, st, block_idx,       \
                     g.cu_seqlens, g.num_seqs, g.total_tokens, g.num_heads, g.block_size, \
                     topk, o_part, lse_part, vmax_bits, out, lse)
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
