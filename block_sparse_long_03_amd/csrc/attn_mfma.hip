// bf16 MFMA block attention for gfx950 (CDNA4), fp32 accumulation.
//
// One tile = up to 128 query rows (4 waves x 32) against a contiguous key
// range of one sequence and head:
//   historical: the gathered queries that selected KV block j, all B keys of
//               block j, no mask ("MoBA: Learned Block Sparsity for
//               Long-Context Attention", "Efficiency and Implementation":
//               queries arranged per selected KV block);
//   own block:  consecutive queries of block c, keys [cB, t], causal mask
//               inside the block (same page, "The Change", causality rule);
//   dense:      consecutive queries, keys [0, t] (the exact baseline of
//               "Starting Point: Exact Softmax Attention and Its Cost").
//
// Per 32-key step each wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16
// (A = 32 keys x 16 dims from LDS, B = the wave's 32 queries from registers),
// so every lane owns one query column and 16 of the 32 keys; the softmax
// statistics need one cross-lane exchange (lane ^ 32).  The probabilities are
// rounded to bf16 in place and used directly as the B operand of
// O^T += V^T P^T; V^T comes from a staging copy whose key order inside each
// group of 16 matches the MFMA output rows, so both operands are single
// 16-byte LDS reads.  K and V^T chunks of 64 keys are double-buffered in LDS
// and prefetched through registers while the previous chunk is computed.
#include "common.h"
#include "launch.h"

namespace moba {

enum { kModeHist = 0, kModeOwn = 1, kModeDense = 2 };

struct MfmaArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* vt;
  const int32_t* cu_seqlens;
  const int32_t* cu_blocks;
  int num_seqs, total_tokens, H, block_size, topk, NB;
  int tiles_per_unit;  // own: query tiles per block; dense: query tiles per sequence
  int units_per_seq;   // own: max blocks per sequence
  float scale2;        // softmax scale * log2(e)
  const int32_t* list;
  const int32_t* offsets;
  const int32_t* tile_offsets;
  void* o_out;  // hist/own: bf16 partials [T, H, topk, D]; dense: out [T, H, D]
  float* lse_out;
};

constexpr int kTK = 64;     // keys per LDS chunk
constexpr int kWaves = 4;

template <int D, int MODE, bool OUT_BF16>
__global__ __launch_bounds__(256, 2) void attn_mfma_kernel(MfmaArgs a) {
  constexpr int TQ = kWaves * 32;
  constexpr int KS = D / 16;   // MFMA k-steps of the QK^T product
  constexpr int DT = D / 32;   // 32-row tiles of O^T
  constexpr int KROW = D + 8;  // LDS row strides in bf16 elements (16 B pad)
  constexpr int VROW = kTK + 8;
  constexpr int KSEG = kTK * D / 8 / 256;  // 16-byte segments per thread per chunk
  constexpr int VSEG = D * kTK / 8 / 256;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kTK * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][D * VROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  // ---------------- tile decode ----------------
  int h, seq_start, seq_len, key_lo, key_hi, gb_base;
  int qtok = -1, qpos = 0x7fffffff;
  long long oidx = 0;
  if (MODE == kModeHist) {
    const int nkeys = a.H * a.NB;
    const int tile = blockIdx.x;
    if (tile >= a.tile_offsets[nkeys]) return;
    const int key = upper_index(a.tile_offsets, nkeys, tile);
    h = key / a.NB;
    const int gb = key - h * a.NB;
    const int s = seq_of_block(a.cu_blocks, a.num_seqs, gb);
    seq_span(a.cu_seqlens, s, a.total_tokens, &seq_start, &seq_len);
    gb_base = a.cu_blocks[s];
    key_lo = (gb - gb_base) * a.block_size;
    key_hi = min(key_lo + a.block_size, seq_len);
    const int e0 = a.offsets[key] + (tile - a.tile_offsets[key]) * TQ;
    const int e1 = min(a.offsets[key + 1], e0 + TQ);
    const int j = e0 + w * 32 + l32;
    if (j < e1) {
      const int ent = a.list[j];
      qtok = ent / a.topk;
      oidx = ((long long)qtok * a.H + h) * a.topk + (ent - qtok * a.topk);
    }
  } else {
    h = blockIdx.y;
    const int per_seq = a.tiles_per_unit * a.units_per_seq;
    const int s = blockIdx.x / per_seq;
    const int rem = per_seq - 1 - (int)(blockIdx.x % per_seq);  // heavy tiles first
    seq_span(a.cu_seqlens, s, a.total_tokens, &seq_start, &seq_len);
    gb_base = a.cu_blocks[s];
    int q_lo, q_hi;
    if (MODE == kModeOwn) {
      const int c = rem / a.tiles_per_unit;
      const int sub = rem % a.tiles_per_unit;
      const int blo = c * a.block_size;
      q_lo = blo + sub * TQ;
      q_hi = min(min(q_lo + TQ, blo + a.block_size), seq_len);
      key_lo = blo;
    } else {
      q_lo = rem * TQ;
      q_hi = min(q_lo + TQ, seq_len);
      key_lo = 0;
    }
    if (q_lo >= q_hi) return;
    key_hi = q_hi;
    const int p = q_lo + w * 32 + l32;
    if (p < q_hi) {
      qtok = seq_start + p;
      qpos = p;
      oidx = (MODE == kModeOwn) ? ((long long)qtok * a.H + h) * a.topk + (a.topk - 1)
                                : (long long)qtok * a.H + h;
    }
  }
  const bool qvalid = qtok >= 0;
  // wave-level query extent (for chunk skipping and masking)
  const uint64_t any_valid = __ballot(qvalid);
  int wq_min = qvalid ? qpos : 0x7fffffff;
  int wq_max = qvalid ? qpos : -1;
  for (int o = 32; o >= 1; o >>= 1) {
    wq_min = min(wq_min, __shfl_xor(wq_min, o));
    wq_max = max(wq_max, __shfl_xor(wq_max, o));
  }

  // ---------------- Q fragments (B operand) ----------------
  bf16x8 qreg[KS];
  {
    const uint16_t* qp = a.q + ((size_t)(qvalid ? qtok : 0) * a.H + h) * D + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 wv = {0u, 0u, 0u, 0u};
      if (qvalid) wv = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
      qreg[ks] = __builtin_bit_cast(bf16x8, wv);
    }
  }

  // ---------------- chunk loader ----------------
  const int nchunks = (key_hi - key_lo + kTK - 1) / kTK;
  u32x4 kbuf[KSEG], vbuf[VSEG];
  auto load_chunk = [&](int ch) {
    const int kp0 = key_lo + ch * kTK;
#pragma unroll
    for (int i = 0; i < KSEG; ++i) {
      const int seg = tid + 256 * i;
      const int r = seg / (D / 8), c = seg % (D / 8);
      const int kp = kp0 + r;
      u32x4 wv = {0u, 0u, 0u, 0u};
      if (kp < seq_len)
        wv = *reinterpret_cast<const u32x4*>(a.k + ((size_t)(seq_start + kp) * a.H + h) * D + c * 8);
      kbuf[i] = wv;
    }
    const int gb = gb_base + kp0 / a.block_size;
    const int off = kp0 % a.block_size;
    const bool gb_ok = gb < a.NB;
    const uint16_t* vb = a.vt + ((size_t)(gb_ok ? gb : 0) * a.H + h) * D * (size_t)a.block_size + off;
#pragma unroll
    for (int i = 0; i < VSEG; ++i) {
      const int seg = tid + 256 * i;
      const int r = seg / (kTK / 8), c = seg % (kTK / 8);
      u32x4 wv = {0u, 0u, 0u, 0u};
      if (gb_ok) wv = *reinterpret_cast<const u32x4*>(vb + (size_t)r * a.block_size + c * 8);
      vbuf[i] = wv;
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KSEG; ++i) {
      const int seg = tid + 256 * i;
      const int r = seg / (D / 8), c = seg % (D / 8);
      *reinterpret_cast<u32x4*>(&Ks[buf][r * KROW + c * 8]) = kbuf[i];
    }
#pragma unroll
    for (int i = 0; i < VSEG; ++i) {
      const int seg = tid + 256 * i;
      const int r = seg / (kTK / 8), c = seg % (kTK / 8);
      *reinterpret_cast<u32x4*>(&Vs[buf][r * VROW + c * 8]) = vbuf[i];
    }
  };

  // ---------------- main loop ----------------
  f32x16 O[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float scale2 = a.scale2;

  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  for (int ch = 0; ch < nchunks; ++ch) {
    const int buf = ch & 1;
    if (ch + 1 < nchunks) load_chunk(ch + 1);
    const int kp0 = key_lo + ch * kTK;
    const bool active = any_valid != 0 && kp0 <= wq_max;
    if (active) {
      const bool need_mask = MODE != kModeHist && kp0 + kTK - 1 > wq_min;
#pragma unroll
      for (int sc = 0; sc < 2; ++sc) {
        f32x16 S;
#pragma unroll
        for (int r = 0; r < 16; ++r) S[r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Ks[buf][(32 * sc + l32) * KROW + 16 * ks + 8 * hf]);
          S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ks], S, 0, 0, 0);
        }
        // S[r] is the score of query (lane & 31) with key
        //   kp0 + 32 sc + 8 (r / 4) + 4 hf + (r % 4)
        if (need_mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kpos = kp0 + 32 * sc + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (kpos > qpos) S[r] = -INFINITY;
          }
        }
        float mx = S[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx * scale2);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        float ls = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = __builtin_amdgcn_exp2f(fmaf(S[r], scale2, -m_use));
          S[r] = p;
          ls += p;
        }
        l_run = l_run * alpha + ls;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) O[dt][r] *= alpha;
        bf16x8 P[2];
#pragma unroll
        for (int mm = 0; mm < 2; ++mm)
#pragma unroll
          for (int i = 0; i < 8; ++i) P[mm][i] = (__bf16)S[8 * mm + i];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) {
            const bf16x8 va = *reinterpret_cast<const bf16x8*>(&Vs[buf][(32 * dt + l32) * VROW + 32 * sc + 16 * mm + 8 * hf]);
            O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, P[mm], O[dt], 0, 0, 0);
          }
        }
      }
    }
    if (ch + 1 < nchunks) store_chunk(buf ^ 1);
    __syncthreads();
  }

  // ---------------- epilogue ----------------
  if (!qvalid) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  const float lse_val = (m_run + log2f(l_tot)) * kLn2;
  // O[dt][r] is output dim 32 dt + 8 (r / 4) + 4 hf + (r % 4) of query (lane & 31)
  if (MODE == kModeDense && !OUT_BF16) {
    float* op = (float*)a.o_out + (size_t)oidx * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v4 = {O[dt][4 * g] * inv, O[dt][4 * g + 1] * inv, O[dt][4 * g + 2] * inv,
                    O[dt][4 * g + 3] * inv};
        *reinterpret_cast<f32x4*>(op + 32 * dt + 8 * g + 4 * hf) = v4;
      }
  } else {
    uint16_t* op = (uint16_t*)a.o_out + (size_t)oidx * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 v2 = {pack_bf16x2(O[dt][4 * g] * inv, O[dt][4 * g + 1] * inv),
                    pack_bf16x2(O[dt][4 * g + 2] * inv, O[dt][4 * g + 3] * inv)};
        *reinterpret_cast<u32x2*>(op + 32 * dt + 8 * g + 4 * hf) = v2;
      }
  }
  if (hf == 0) a.lse_out[oidx] = lse_val;
}

static MfmaArgs base_args(const void* q, const void* k, const uint16_t* vt, const Geo& g,
                          int topk, float scale) {
  MfmaArgs a{};
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.vt = vt;
  a.cu_seqlens = g.cu_seqlens;
  a.cu_blocks = g.cu_blocks;
  a.num_seqs = g.num_seqs;
  a.total_tokens = g.total_tokens;
  a.H = g.num_heads;
  a.block_size = g.block_size;
  a.topk = topk;
  a.NB = g.total_blocks;
  a.scale2 = scale * kLog2e;
  return a;
}

hipError_t launch_attn_mfma_hist(const void* q, const void* k, const uint16_t* vt,
                                 const Geo& g, int topk, float scale, const int32_t* list,
                                 const int32_t* offsets, const int32_t* tile_offsets,
                                 long long max_tiles, uint16_t* o_part, float* lse_part,
                                 hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
  MfmaArgs a = base_args(q, k, vt, g, topk, scale);
  a.list = list;
  a.offsets = offsets;
  a.tile_offsets = tile_offsets;
  a.o_out = o_part;
  a.lse_out = lse_part;
  dim3 grid((unsigned)max_tiles);
  if (g.head_dim == 128)
    hipLaunchKernelGGL((attn_mfma_kernel<128, kModeHist, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<64, kModeHist, true>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_mfma_own(const void* q, const void* k, const uint16_t* vt,
                                const Geo& g, int topk, float scale, uint16_t* o_part,
                                float* lse_part, hipStream_t st) {
  if (g.total_tokens == 0 || g.max_seqlen == 0) return hipSuccess;
  MfmaArgs a = base_args(q, k, vt, g, topk, scale);
  a.tiles_per_unit = (g.block_size + kMfmaTileQ - 1) / kMfmaTileQ;
  a.units_per_seq = (g.max_seqlen + g.block_size - 1) / g.block_size;
  a.o_out = o_part;
  a.lse_out = lse_part;
  dim3 grid((unsigned)(g.num_seqs * a.tiles_per_unit * a.units_per_seq), g.num_heads);
  if (g.head_dim == 128)
    hipLaunchKernelGGL((attn_mfma_kernel<128, kModeOwn, true>), grid, dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<64, kModeOwn, true>), grid, dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_mfma_dense(const void* q, const void* k, const uint16_t* vt,
                                  const Geo& g, float scale, void* out, bool out_bf16,
                                  float* lse, hipStream_t st) {
  if (g.total_tokens == 0 || g.max_seqlen == 0) return hipSuccess;
  MfmaArgs a = base_args(q, k, vt, g, 1, scale);
  a.tiles_per_unit = (g.max_seqlen + kMfmaTileQ - 1) / kMfmaTileQ;
  a.units_per_seq = 1;
  a.o_out = out;
  a.lse_out = lse;
  dim3 grid((unsigned)(g.num_seqs * a.tiles_per_unit), g.num_heads);
#define MOBA_DENSE(D, OB) \
  hipLaunchKernelGGL((attn_mfma_kernel<D, kModeDense, OB>), grid, dim3(256), 0, st, a)
  if (g.head_dim == 128) { if (out_bf16) MOBA_DENSE(128, true); else MOBA_DENSE(128, false); }
  else { if (out_bf16) MOBA_DENSE(64, true); else MOBA_DENSE(64, false); }
#undef MOBA_DENSE
  return hipGetLastError();
}

}  // namespace moba
