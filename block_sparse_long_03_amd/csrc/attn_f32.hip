// fp32 attention for fp32 inputs (small, high-precision runs).  One wave per
// (query row, key range); the lanes split the head dimension and every score
// is a wave-wide fp32 dot product; online softmax in natural exp.
// Same decomposition as the bf16 path: historical partials from the per-block
// query lists, own-block causal partials, then the shared merge kernel
// ("MoBA: Learned Block Sparsity for Long-Context Attention", "Efficiency and
// Implementation"); dense causal rows write the final output directly.
#include "common.h"
#include "launch.h"

namespace moba {

template <int D>
__device__ __forceinline__ void attend_range_f32(const float* __restrict__ q,
                                                 const float* __restrict__ k,
                                                 const float* __restrict__ v, int H, int h,
                                                 int qtok, int seq_start, int key_lo,
                                                 int key_hi, float scale, float* o,
                                                 float* lse_out) {
  constexpr int PER = D / 64;
  const int lane = threadIdx.x & 63;
  float qv[PER], acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    qv[e] = q[((size_t)qtok * H + h) * D + lane * PER + e];
    acc[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int j = key_lo; j < key_hi; ++j) {
    const size_t row = ((size_t)(seq_start + j) * H + h) * D + lane * PER;
    float part = 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) part = fmaf(qv[e], k[row + e], part);
    const float x = wave_sum(part) * scale;
    const float m_new = fmaxf(m, x);
    const float alpha = expf(m - m_new);
    const float p = expf(x - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = fmaf(p, v[row + e], acc[e] * alpha);
    m = m_new;
  }
  const float inv = 1.f / l;
#pragma unroll
  for (int e = 0; e < PER; ++e) o[lane * PER + e] = acc[e] * inv;
  if (lane == 0) *lse_out = m + logf(l);
}

// historical partials: one wave per list entry.  Lists and partials cover the
// HC heads h0 .. h0 + HC - 1 (indexed by the place in the group); q, k, v
// rows have H heads.
template <int D>
__global__ __launch_bounds__(256) void attn_f32_hist_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ cu_seqlens, const int32_t* __restrict__ cu_blocks,
    int num_seqs, int total_tokens, int H, int h0, int HC, int NB, int block_size, int topk,
    float scale, const int32_t* __restrict__ list, const int32_t* __restrict__ offsets,
    float* __restrict__ o_part, float* __restrict__ lse_part) {
  const int nkeys = HC * NB;
  const long long e = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= offsets[nkeys]) return;
  const int key = upper_index(offsets, nkeys, (int)e);
  const int h = key / NB;
  const int gb = key - h * NB;
  const int s = seq_of_block(cu_blocks, num_seqs, gb);
  int start, len;
  seq_span(cu_seqlens, s, total_tokens, &start, &len);
  const int lo = (gb - cu_blocks[s]) * block_size;
  const int hi = min(lo + block_size, len);
  const int ent = list[e];
  const int t = ent / topk;
  const size_t oi = ((size_t)t * HC + h) * topk + (ent - t * topk);
  attend_range_f32<D>(q, k, v, H, h0 + h, t, start, lo, hi, scale, o_part + oi * D,
                      lse_part + oi);
}

// own-block partials (mode 0, rows of the HC heads h0 .. h0 + HC - 1, partials
// indexed by the place in the group) or dense causal output (mode 1, every
// head: h0 = 0, HC = H): one wave per row
template <int D, int MODE, bool OUT_BF16>
__global__ __launch_bounds__(256) void attn_f32_rows_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const int32_t* __restrict__ cu_seqlens, int num_seqs, int total_tokens, int H, int h0,
    int HC, int block_size, int topk, float scale, float* __restrict__ o_part,
    float* __restrict__ lse_part, void* __restrict__ out, float* __restrict__ lse) {
  __shared__ float obuf[4][D];
  const int wv = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * 4 + wv;
  if (row >= (long long)total_tokens * HC) return;
  const int t = (int)(row / HC);
  const int h = h0 + (int)(row - (long long)t * HC);
  const int s = upper_index(cu_seqlens, num_seqs, t);
  const int start = cu_seqlens[s];
  const int p = t - start;
  if (MODE == 0) {
    const int lo = (p / block_size) * block_size;
    const size_t oi = (size_t)row * topk + (topk - 1);
    attend_range_f32<D>(q, k, v, H, h, t, start, lo, p + 1, scale, o_part + oi * D,
                        lse_part + oi);
  } else {
    attend_range_f32<D>(q, k, v, H, h, t, start, 0, p + 1, scale, obuf[wv], lse + row);
    __builtin_amdgcn_wave_barrier();
    const int lane = threadIdx.x & 63;
    for (int e = lane; e < D; e += 64) {
      if (OUT_BF16) ((uint16_t*)out)[(size_t)row * D + e] = f32_to_bf16_bits(obuf[wv][e]);
      else ((float*)out)[(size_t)row * D + e] = obuf[wv][e];
    }
  }
}

hipError_t launch_attn_f32_hist(const float* q, const float* k, const float* v, const Geo& g,
                                int topk, float scale, const int32_t* list,
                                const int32_t* offsets, long long max_entries, float* o_part,
                                float* lse_part, hipStream_t st) {
  if (max_entries <= 0) return hipSuccess;
  dim3 grid((unsigned)((max_entries + 3) / 4));
#define MOBA_F32H(D)                                                                      \
  hipLaunchKernelGGL(attn_f32_hist_kernel<D>, grid, dim3(256), 0, st, q, k, v, g.cu_seqlens, \
                     g.cu_blocks, g.num_seqs, g.total_tokens, g.num_heads, g.head_lo,       \
                     g.head_cnt, g.total_blocks, g.block_size, topk, scale, list, offsets,  \
                     o_part, lse_part)
  if (g.head_dim == 128) MOBA_F32H(128); else MOBA_F32H(64);
#undef MOBA_F32H
  return hipGetLastError();
}

hipError_t launch_attn_f32_own(const float* q, const float* k, const float* v, const Geo& g,
                               int topk, float scale, float* o_part, float* lse_part,
                               hipStream_t st) {
  const long long rows = (long long)g.total_tokens * g.head_cnt;
  if (rows == 0) return hipSuccess;
  dim3 grid((unsigned)((rows + 3) / 4));
  if (g.head_dim == 128)
    hipLaunchKernelGGL((attn_f32_rows_kernel<128, 0, false>), grid, dim3(256), 0, st, q, k, v,
                       g.cu_seqlens, g.num_seqs, g.total_tokens, g.num_heads, g.head_lo,
                       g.head_cnt, g.block_size, topk, scale, o_part, lse_part, nullptr,
                       nullptr);
  else
    hipLaunchKernelGGL((attn_f32_rows_kernel<64, 0, false>), grid, dim3(256), 0, st, q, k, v,
                       g.cu_seqlens, g.num_seqs, g.total_tokens, g.num_heads, g.head_lo,
                       g.head_cnt, g.block_size, topk, scale, o_part, lse_part, nullptr,
                       nullptr);
  return hipGetLastError();
}

hipError_t launch_attn_f32_dense(const float* q, const float* k, const float* v, const Geo& g,
                                 float scale, void* out, bool out_bf16, float* lse,
                                 hipStream_t st) {
  const long long rows = (long long)g.total_tokens * g.num_heads;
  if (rows == 0) return hipSuccess;
  dim3 grid((unsigned)((rows + 3) / 4));
#define MOBA_F32D(D, OB)                                                                   \
  hipLaunchKernelGGL((attn_f32_rows_kernel<D, 1, OB>), grid, dim3(256), 0, st, q, k, v,     \
                     g.cu_seqlens, g.num_seqs, g.total_tokens, g.num_heads, 0, g.num_heads, \
                     g.block_size, 1, scale, nullptr, nullptr, out, lse)
  if (g.head_dim == 128) { if (out_bf16) MOBA_F32D(128, true); else MOBA_F32D(128, false); }
  else { if (out_bf16) MOBA_F32D(64, true); else MOBA_F32D(64, false); }
#undef MOBA_F32D
  return hipGetLastError();
}

}  // namespace moba
