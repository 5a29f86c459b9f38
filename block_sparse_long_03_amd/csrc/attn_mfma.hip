// bf16 MFMA block attention for gfx950 (CDNA4), fp32 accumulation.
//
// One tile = up to 128 or 256 query rows (4 waves x 32 or 64) against a contiguous key
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
// rounded to fp16 in place and used directly as the B operand of
// O^T += V^T P^T (fp16 MFMA: probabilities carry 11 significant bits); V^T
// comes from an fp16 staging copy (exact for bf16 V, scaled per head) whose key order inside each
// group of 16 matches the MFMA output rows, so both operands are single
// 16-byte LDS reads.  K and V^T chunks of 64 keys are double-buffered in LDS
// and prefetched through registers while the previous chunk is computed.
#include "common.h"
#include "launch.h"

namespace moba {

enum { kModeHist = 0, kModeOwn = 1, kModeDense = 2 };

// max / sum of a value and the same register of lane (lane ^ 32): one
// v_permlane32_swap, which hands each half the other half's value
__device__ __forceinline__ float max_with_partner(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

struct MfmaArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* vt;          // fp16 V^T staging copy, scaled per head by 2^-e
  const uint32_t* vmax_bits;   // per-head max |v| (fp32 bits): dense mode scales back
  const int32_t* cu_seqlens;
  const int32_t* cu_blocks;
  int num_seqs, total_tokens, H, block_size, topk, NB;
  int tiles_per_unit;  // own: query tiles per block; dense: query tiles per sequence
  int units_per_seq;   // own: max blocks per sequence
  float scale2;        // softmax scale * log2(e)
  const int32_t* list;
  const int4* tile_info;  // hist: {key, first entry, end entry, 0} per tile, key < 0 past the end
  void* o_out;  // hist/own: fp16 partials [T, H, topk, D] (V units); dense: out [T, H, D]
  float* lse_out;
};

constexpr int kTK = 64;     // keys per LDS chunk
constexpr int kWaves = kMfmaWaves;
constexpr int kThreads = 64 * kWaves;
constexpr int kQT = kMfmaTileQ / (kWaves * 32);  // 32-query column tiles per wave
// Lazy rescaling: the running max used as the exponent base only moves when a
// new score exceeds it by more than 2^8, so the O accumulators are rescaled
// rarely; probabilities stay below 256 (exact in the final normalisation).
constexpr float kRescaleSlack = 8.0f;

template <int D, int MODE, bool OUT_BF16, int QT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kMfmaWavesPerSimd)))
void attn_mfma_kernel(MfmaArgs a) {
  constexpr int TQ = kWaves * 32 * QT;
  constexpr int KS = D / 16;   // MFMA k-steps of the QK^T product
  constexpr int DT = D / 32;   // 32-row tiles of O^T
  constexpr int KROW = D + 8;  // LDS row strides in bf16 elements (16 B pad)
  constexpr int VROW = kTK + 8;
  constexpr int NSEG = kTK * D / 8;  // 16-byte segments of a K (or V^T) chunk
  constexpr int KSEG = (NSEG + kThreads - 1) / kThreads;  // per thread
  constexpr int VSEG = KSEG;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2][kTK * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Vs[2][D * VROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  // ---------------- tile decode ----------------
  int h, seq_start, seq_len, key_lo, key_hi, gb_base;
  int qtok[QT], qpos[QT];
  long long oidx[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) { qtok[qt] = -1; qpos[qt] = 0x7fffffff; oidx[qt] = 0; }
  if (MODE == kModeHist) {
    const int4 ti = a.tile_info[blockIdx.x];
    const int key = ti.x;
    if (key < 0) return;
    h = key / a.NB;
    const int gb = key - h * a.NB;
    const int s = seq_of_block(a.cu_blocks, a.num_seqs, gb);
    seq_span(a.cu_seqlens, s, a.total_tokens, &seq_start, &seq_len);
    gb_base = a.cu_blocks[s];
    key_lo = (gb - gb_base) * a.block_size;
    key_hi = min(key_lo + a.block_size, seq_len);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int j = ti.y + (w * QT + qt) * 32 + l32;
      if (j < ti.z) {
        const int ent = a.list[j];
        qtok[qt] = ent / a.topk;
        oidx[qt] = ((long long)qtok[qt] * a.H + h) * a.topk + (ent - qtok[qt] * a.topk);
      }
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
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int p = q_lo + (w * QT + qt) * 32 + l32;
      if (p < q_hi) {
        qtok[qt] = seq_start + p;
        qpos[qt] = p;
        oidx[qt] = (MODE == kModeOwn) ? ((long long)qtok[qt] * a.H + h) * a.topk + (a.topk - 1)
                                      : (long long)qtok[qt] * a.H + h;
      }
    }
  }
  // smallest query position of the wave: chunks past it need the causal mask
  int wq_min = 0x7fffffff;
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
    if (qtok[qt] >= 0) wq_min = min(wq_min, qpos[qt]);
  for (int o = 32; o >= 1; o >>= 1) wq_min = min(wq_min, __shfl_xor(wq_min, o));

  // ---------------- Q fragments (B operand) ----------------
  bf16x8 qreg[QT][KS];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const bool qv = qtok[qt] >= 0;
    const uint16_t* qp = a.q + ((size_t)(qv ? qtok[qt] : 0) * a.H + h) * D + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 wv = {0u, 0u, 0u, 0u};
      if (qv) wv = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
      qreg[qt][ks] = __builtin_bit_cast(bf16x8, wv);
    }
  }

  // ---------------- chunk loader ----------------
  // Every thread moves the same 16-byte segments of each chunk; the per-chunk
  // base addresses are wave-uniform, the per-thread offsets fixed 32-bit values.
  const int nchunks = (key_hi - key_lo + kTK - 1) / kTK;
  const size_t krow_bytes = (size_t)a.H * D * 2;
  const char* kseq = (const char*)a.k + ((size_t)seq_start * a.H + h) * D * 2;
  uint32_t koff[KSEG], voff[VSEG];
  int krow[KSEG];
#pragma unroll
  for (int i = 0; i < KSEG; ++i) {
    const int seg = min(tid + kThreads * i, NSEG - 1);
    krow[i] = seg / (D / 8);
    koff[i] = (uint32_t)(krow[i] * krow_bytes + (seg % (D / 8)) * 16);
  }
#pragma unroll
  for (int i = 0; i < VSEG; ++i) {
    const int seg = min(tid + kThreads * i, NSEG - 1);
    voff[i] = (uint32_t)(((seg / (kTK / 8)) * a.block_size + (seg % (kTK / 8)) * 8) * 2);
  }
  // V^T source of the next chunk to load: block gb_next at offset off_next
  int gb_next = gb_base + key_lo / a.block_size;
  int off_next = key_lo % a.block_size;
  u32x4 kbuf[KSEG], vbuf[VSEG];
  auto load_chunk = [&](int ch) {
    const int kp0 = key_lo + ch * kTK;
    const char* kb = kseq + (size_t)kp0 * krow_bytes;
    if (kp0 + kTK <= seq_len) {
#pragma unroll
      for (int i = 0; i < KSEG; ++i) kbuf[i] = *reinterpret_cast<const u32x4*>(kb + koff[i]);
    } else {
#pragma unroll
      for (int i = 0; i < KSEG; ++i) {
        u32x4 wv = {0u, 0u, 0u, 0u};
        if (kp0 + krow[i] < seq_len) wv = *reinterpret_cast<const u32x4*>(kb + koff[i]);
        kbuf[i] = wv;
      }
    }
    if (gb_next < a.NB) {
      const char* vb =
          (const char*)(a.vt + ((size_t)gb_next * a.H + h) * D * (size_t)a.block_size + off_next);
#pragma unroll
      for (int i = 0; i < VSEG; ++i) vbuf[i] = *reinterpret_cast<const u32x4*>(vb + voff[i]);
    } else {
#pragma unroll
      for (int i = 0; i < VSEG; ++i) vbuf[i] = u32x4{0u, 0u, 0u, 0u};
    }
    off_next += kTK;
    if (off_next == a.block_size) { off_next = 0; ++gb_next; }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KSEG; ++i) {
      const int seg = tid + kThreads * i;
      if (NSEG % kThreads == 0 || seg < NSEG) {
        const int r = seg / (D / 8), c = seg % (D / 8);
        *reinterpret_cast<u32x4*>(&Ks[buf][r * KROW + c * 8]) = kbuf[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VSEG; ++i) {
      const int seg = tid + kThreads * i;
      if (NSEG % kThreads == 0 || seg < NSEG) {
        const int r = seg / (kTK / 8), c = seg % (kTK / 8);
        *reinterpret_cast<u32x4*>(&Vs[buf][r * VROW + c * 8]) = vbuf[i];
      }
    }
  };

  // ---------------- main loop ----------------
  // Software pipeline over 32-key steps: the QK^T product of the next step is
  // issued while the probabilities of the current step are formed, and the
  // current PV product runs while the next step's row max is taken, so the
  // matrix cores and the vector ALUs of a wave work side by side.
  static_assert(QT == 1, "one 32-query column tile per wave");
  f32x16 O[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[dt][r] = 0.f;
  float m_use = -INFINITY, l_run = 0.f;
  const float scale2 = a.scale2;
  const int qp = qpos[0];

  auto qk = [&](int buf, int sc) {
    f32x16 S;
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&Ks[buf][(32 * sc + l32) * KROW + 16 * ks + 8 * hf]);
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[0][ks], S, 0, 0, 0);
    }
    return S;
  };
  // S[r] is the score of query column (lane & 31) with key kp + 8 (r / 4) + 4 hf + (r % 4)
  auto mask = [&](f32x16& S, int kp) {
    if (MODE != kModeHist && kp + 31 > wq_min) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kp + 8 * (r >> 2) + 4 * hf + (r & 3) > qp) S[r] = -INFINITY;
    }
  };
  auto row_max = [&](const f32x16& S) {
    float mx = S[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, S[r]);
    return max_with_partner(mx);
  };
  auto rescale = [&](float mx) {
    const float cand = mx * scale2;
    if (__ballot(cand > m_use + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_use, cand);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_use - m_new);
      m_use = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[dt][r] *= alpha;
    }
  };
  auto probs = [&](f32x16 S, f16x8* P) {
    const float base = m_use == -INFINITY ? 0.f : m_use;
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = __builtin_amdgcn_exp2f(fmaf(S[r], scale2, -base));
#pragma unroll
    for (int mm = 0; mm < 2; ++mm)
#pragma unroll
      for (int i = 0; i < 8; ++i) P[mm][i] = (_Float16)S[8 * mm + i];
    float ls = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) ls += S[r];
    l_run += ls;
  };
  auto pv = [&](int buf, int sc, const f16x8* P) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const f16x8 va = *reinterpret_cast<const f16x8*>(&Vs[buf][(32 * dt + l32) * VROW + 32 * sc + 16 * mm + 8 * hf]);
        O[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(va, P[mm], O[dt], 0, 0, 0);
      }
  };

  load_chunk(0);
  store_chunk(0);
  if (nchunks > 1) load_chunk(1);
  __syncthreads();
  f32x16 Sa = qk(0, 0);
  mask(Sa, key_lo);
  rescale(row_max(Sa));
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    const int kp0 = key_lo + c * kTK;
    f16x8 P[2];
    // first 32 keys of chunk c; the QK^T of its second 32 keys is in flight
    f32x16 Sb = qk(buf, 1);
    probs(Sa, P);
    pv(buf, 0, P);
    mask(Sb, kp0 + 32);
    const float mxb = row_max(Sb);
    if (c + 1 < nchunks) store_chunk(buf ^ 1);
    __syncthreads();  // chunk c + 1 is in LDS
    if (c + 2 < nchunks) load_chunk(c + 2);
    rescale(mxb);
    // second 32 keys of chunk c; the QK^T of chunk c + 1's first 32 keys is in
    // flight (on the last chunk it reads a stale buffer and is discarded)
    Sa = qk(buf ^ 1, 0);
    probs(Sb, P);
    pv(buf, 1, P);
    if (c + 1 < nchunks) {
      mask(Sa, kp0 + kTK);
      rescale(row_max(Sa));
    }
    __syncthreads();  // every wave is done with chunk c's buffer
  }

  // ---------------- epilogue ----------------
  float out_scale = 1.f;
  if (MODE == kModeDense) out_scale = __builtin_ldexpf(1.0f, v_exponent(a.vmax_bits[h]));
  {
    constexpr int qt = 0;
    // both lanes of a query column take the same branch
    if (qtok[qt] < 0) return;
    const float l_tot = sum_with_partner(l_run);
    const float inv = out_scale / l_tot;
    const float lse_val = (m_use + log2f(l_tot)) * kLn2;
    // O[dt][r] is output dim 32 dt + 8 (r / 4) + 4 hf + (r % 4)
    if (MODE == kModeDense && !OUT_BF16) {
      float* op = (float*)a.o_out + (size_t)oidx[qt] * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v4 = {O[dt][4 * g] * inv, O[dt][4 * g + 1] * inv,
                      O[dt][4 * g + 2] * inv, O[dt][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(op + 32 * dt + 8 * g + 4 * hf) = v4;
        }
    } else if (MODE == kModeDense) {
      uint16_t* op = (uint16_t*)a.o_out + (size_t)oidx[qt] * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 v2 = {pack_bf16x2(O[dt][4 * g] * inv, O[dt][4 * g + 1] * inv),
                      pack_bf16x2(O[dt][4 * g + 2] * inv, O[dt][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(op + 32 * dt + 8 * g + 4 * hf) = v2;
        }
    } else {
      uint16_t* op = (uint16_t*)a.o_out + (size_t)oidx[qt] * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x2 v2 = {pack_f16x2(O[dt][4 * g] * inv, O[dt][4 * g + 1] * inv),
                      pack_f16x2(O[dt][4 * g + 2] * inv, O[dt][4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(op + 32 * dt + 8 * g + 4 * hf) = v2;
        }
    }
    if (hf == 0) a.lse_out[oidx[qt]] = lse_val;
  }
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
                                 const int4* tile_info, long long max_tiles, uint16_t* o_part,
                                 float* lse_part, hipStream_t st) {
  if (max_tiles <= 0) return hipSuccess;
  MfmaArgs a = base_args(q, k, vt, g, topk, scale);
  a.list = list;
  a.tile_info = tile_info;
  a.o_out = o_part;
  a.lse_out = lse_part;
  dim3 grid((unsigned)max_tiles);
  if (g.head_dim == 128)
    hipLaunchKernelGGL((attn_mfma_kernel<128, kModeHist, true, kQT>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<64, kModeHist, true, kQT>), grid, dim3(kThreads), 0, st, a);
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
    hipLaunchKernelGGL((attn_mfma_kernel<128, kModeOwn, true, kQT>), grid, dim3(kThreads), 0, st, a);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<64, kModeOwn, true, kQT>), grid, dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_mfma_dense(const void* q, const void* k, const uint16_t* vt,
                                  const uint32_t* vmax_bits, const Geo& g, float scale,
                                  void* out, bool out_bf16, float* lse, hipStream_t st) {
  if (g.total_tokens == 0 || g.max_seqlen == 0) return hipSuccess;
  MfmaArgs a = base_args(q, k, vt, g, 1, scale);
  a.vmax_bits = vmax_bits;
  a.tiles_per_unit = (g.max_seqlen + kMfmaTileQ - 1) / kMfmaTileQ;
  a.units_per_seq = 1;
  a.o_out = out;
  a.lse_out = lse;
  dim3 grid((unsigned)(g.num_seqs * a.tiles_per_unit), g.num_heads);
#define MOBA_DENSE(D, OB) \
  hipLaunchKernelGGL((attn_mfma_kernel<D, kModeDense, OB, kQT>), grid, dim3(kThreads), 0, st, a)
  if (g.head_dim == 128) { if (out_bf16) MOBA_DENSE(128, true); else MOBA_DENSE(128, false); }
  else { if (out_bf16) MOBA_DENSE(64, true); else MOBA_DENSE(64, false); }
#undef MOBA_DENSE
  return hipGetLastError();
}

}  // namespace moba
