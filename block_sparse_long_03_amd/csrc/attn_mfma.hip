// bf16 MFMA block attention for gfx950 (CDNA4), fp32 accumulation.
//
// One tile = up to 128 or 256 query rows (4 or 8 waves x 32) against a contiguous key
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
// comes from an fp16 staging copy (exact for bf16 V, scaled per head) whose
// key order inside each group of 16 matches the MFMA output rows, so both
// operands are single 16-byte LDS reads.
//
// K and V^T chunks of 64 keys are double-buffered in LDS and filled by direct
// global-to-LDS loads (buffer_load_dwordx4 ... lds: each wave instruction
// writes 1 KiB of consecutive LDS, no registers involved) while the previous chunk
// is computed; one barrier per chunk (8-wave dense tiles: four slots, one
// barrier per two chunks).  When a whole block fits in LDS
// (B * d * 4 bytes <= 128 KiB), historical tiles keep it resident instead:
// every chunk is loaded once, and each wave then runs several passes of 32
// gathered queries over the resident chunks with no further barrier.  The LDS tiles are unpadded and
// XOR-swizzled in 16-byte segments so that the MFMA operand reads are free of
// bank conflicts: rows of 256 B use segment ^ (row & 15), rows of 128 B use
// segment ^ ((row >> 1) & 7).  Output rows leave through a 4 KiB LDS tile
// per wave so that they are stored as whole 128-byte lines.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moba {

// kModeHistRes: historical tiles with the whole KV block resident in LDS
enum { kModeHist = 0, kModeOwn = 1, kModeDense = 2, kModeHistRes = 3 };

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
  // H: heads of the group this launch covers (the head index h below is a
  // place in it; partials and staged V are laid out for H heads); Hs: heads
  // of the q/k (and dense out/lse) rows; h0: global head of place 0
  int num_seqs, total_tokens, H, Hs, h0, block_size, topk, NB;
  int tiles_per_unit;  // own: query tiles per block; dense: query tiles per sequence
  int units_per_seq;   // own: max blocks per sequence
  int q_limit;         // dense: queries at local positions below it only
  int dense_blocks;    // own: blocks below it whose notfull flag is 0 are skipped
  const int32_t* notfull;
  float scale2;        // softmax scale * log2(e)
  uint32_t topk_magic; // floor((2^32 - 1) / topk): list entries split without a division
  const int32_t* list;
  const int4* tile_info;  // hist: {key, first entry, end entry, 0} per tile, key < 0 past the end
  void* o_out;  // hist/own: fp16 partials [T, H, topk, D] (V units); dense: out [T, Hs, D]
  float* lse_out;
};

constexpr int kTK = 64;     // keys per LDS chunk

// segment swizzle of an LDS tile row (row_bytes 256 or 128)
template <int ROW_BYTES>
__device__ __forceinline__ int swz(int row) {
  return ROW_BYTES == 256 ? (row & 15) : ((row >> 1) & 7);
}

// Lazy rescaling: the running max used as the exponent base of a query only
// moves when one of its new scores exceeds it by more than 2^8, so the O
// accumulators are rescaled rarely; probabilities stay below 256 (exact in
// the final normalisation).  The decision is taken per query column (the two
// lanes of a column agree), never per wave, so a query's rounding is the same
// whichever queries share its wave and the forward is bitwise reproducible
// even though the order of the bucket lists is not.
constexpr float kRescaleSlack = 8.0f;

template <int D, int MODE, bool OUT_BF16, int kWaves>
__global__ __launch_bounds__(64 * kWaves) __attribute__((amdgpu_waves_per_eu(kMfmaWavesPerSimd)))
void attn_mfma_kernel(MfmaArgs a) {
  constexpr int TQ = kWaves * 32;
  constexpr int KS = D / 16;             // MFMA k-steps of the QK^T product
  constexpr int DT = D / 32;             // 32-row tiles of O^T
  constexpr int KRB = D * 2;             // bytes of a K row in LDS (256 / 128)
  constexpr int VRB = kTK * 2;           // bytes of a V^T row in LDS (128)
  constexpr int KBYTES = kTK * KRB;      // one K chunk
  constexpr int VBYTES = D * VRB;        // one V^T chunk
  constexpr int BUF = KBYTES + VBYTES;
  constexpr int NKI = KBYTES / 1024;     // 1-KiB wave loads per K chunk
  constexpr int NVI = VBYTES / 1024;
  constexpr int KIW = (NKI + kWaves - 1) / kWaves;  // per wave
  constexpr int VIW = (NVI + kWaves - 1) / kWaves;
  constexpr bool RES = MODE == kModeHistRes;
  constexpr bool HIST = MODE == kModeHist || RES;
  static_assert(!RES || kWaves == 8, "resident tiles run 8 waves");
  // K/V: the resident block or the two chunk slots; then a 4 KiB output
  // staging tile per wave
  constexpr int kStageBytes = 4096;
  // 8-wave dense tiles: four K/V chunk slots and one barrier per two chunks
  // (1.5-2% faster there; the historical tiles gain nothing from it)
  constexpr bool RING4 = MODE == kModeDense && kWaves == 8;
  constexpr int kStageOff = RES ? kResidentLdsBytes : (RING4 ? 4 : 2) * BUF;
  __shared__ __attribute__((aligned(1024))) char smem[kStageOff + kWaves * kStageBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  // ---------------- tile decode ----------------
  int h, seq_start, seq_len, key_lo, key_hi, gb_base;
  int qtok = -1, qpos = 0x7fffffff;
  long long oidx = 0;
  int4 ti = {0, 0, 0, 0};
  if (HIST) {
    ti = a.tile_info[blockIdx.x];
    const int key = ti.x;
    if (key < 0) return;
    h = key / a.NB;
    const int gb = key - h * a.NB;
    const int s = seq_of_block(a.cu_blocks, a.num_seqs, gb);
    seq_span(a.cu_seqlens, s, a.total_tokens, &seq_start, &seq_len);
    gb_base = a.cu_blocks[s];
    key_lo = (gb - gb_base) * a.block_size;
    key_hi = min(key_lo + a.block_size, seq_len);
    if (!RES) {
      const int j = ti.y + w * 32 + l32;
      if (j < ti.z) {
        const int ent = a.list[j];
        qtok = ent / a.topk;
        oidx = ((long long)qtok * a.H + h) * a.topk + (ent - qtok * a.topk);
      }
    }
  } else {
    // XCD-contiguous order: the tiles of one block (own) or sequence (dense)
    // and head share an L2
    const int L = xcd_remap(blockIdx.x + blockIdx.y * gridDim.x, gridDim.x * gridDim.y);
    const int bx = L % gridDim.x;
    h = L / gridDim.x;
    const int per_seq = a.tiles_per_unit * a.units_per_seq;
    const int s = bx / per_seq;
    const int rem = per_seq - 1 - (bx % per_seq);  // heavy tiles first
    seq_span(a.cu_seqlens, s, a.total_tokens, &seq_start, &seq_len);
    gb_base = a.cu_blocks[s];
    int q_lo, q_hi;
    if (MODE == kModeOwn) {
      const int c = rem / a.tiles_per_unit;
      const int sub = rem % a.tiles_per_unit;
      // every row of a block below dense_blocks with notfull 0 is written by
      // the dense-prefix pass
      if (c < a.dense_blocks && gb_base + c < a.NB &&
          a.notfull[(size_t)h * a.NB + gb_base + c] == 0)
        return;
      const int blo = c * a.block_size;
      q_lo = blo + sub * TQ;
      q_hi = min(min(q_lo + TQ, blo + a.block_size), seq_len);
      key_lo = blo;
    } else {
      q_lo = rem * TQ;
      q_hi = min(min(q_lo + TQ, seq_len), a.q_limit);
      key_lo = 0;
    }
    if (q_lo >= q_hi) return;
    key_hi = q_hi;
    const int p = q_lo + w * 32 + l32;
    if (p < q_hi) {
      qtok = seq_start + p;
      qpos = p;
      oidx = (MODE == kModeOwn) ? ((long long)qtok * a.H + h) * a.topk + (a.topk - 1)
                                : (long long)qtok * a.Hs + a.h0 + h;
    }
  }
  const int hg = a.h0 + h;  // global head of the q/k rows
  // smallest query position of the wave: chunks past it need the causal mask
  int wq_min = qtok >= 0 ? qpos : 0x7fffffff;
  for (int o = 32; o >= 1; o >>= 1) wq_min = min(wq_min, __shfl_xor(wq_min, o));

  // ---------------- Q fragments (B operand) ----------------
  bf16x8 qreg[KS];
  if (!RES) {
    const bool qv = qtok >= 0;
    const uint16_t* qp = a.q + ((size_t)(qv ? qtok : 0) * a.Hs + hg) * D + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 wv = {0u, 0u, 0u, 0u};
      if (qv) wv = *reinterpret_cast<const u32x4*>(qp + 16 * ks);
      qreg[ks] = __builtin_bit_cast(bf16x8, wv);
    }
  }

  // ---------------- chunk loads (global -> LDS) ----------------
  // Wave instruction i of a chunk load fills LDS bytes [(w + kWaves i) KiB,
  // +1 KiB): lane `lane` writes 16 bytes of row r at segment lseg.  Moving
  // to the next instruction adds a whole number of 16-row groups, so the
  // swizzle, and with it the lane's source offset, only shifts by a uniform
  // amount.
  constexpr int KROWS_I = kWaves * 1024 / KRB;  // K rows per wave instruction step
  constexpr int VROWS_I = kWaves * 1024 / VRB;
  static_assert(KROWS_I % 16 == 0 && VROWS_I % 16 == 0, "uniform per-instruction offsets");
  const int nchunks = (key_hi - key_lo + kTK - 1) / kTK;
  const size_t krow_bytes = (size_t)a.Hs * D * 2;
  const char* kseq = (const char*)a.k + ((size_t)seq_start * a.Hs + hg) * D * 2;
  const int krow0 = (w * 1024 + lane * 16) / KRB;
  const uint32_t koff0 = (uint32_t)(krow0 * krow_bytes +
                                    ((((lane * 16) % KRB) >> 4) ^ swz<KRB>(krow0)) * 16);
  const int vrow0 = (w * 1024 + lane * 16) / VRB;
  const uint32_t voff0 = (uint32_t)(vrow0 * a.block_size * 2 +
                                    ((((lane * 16) % VRB) >> 4) ^ swz<VRB>(vrow0)) * 16);
  // One buffer descriptor for the tile's keys, built once: a whole chunk's
  // rows are then reached through the lane's record index (16-byte records,
  // krec of them per key row), with no per-chunk address arithmetic in
  // scalar registers.  Tiles whose key span would take the index past 2^31
  // rebuild the descriptor per chunk instead.
  const uint32_t krec = (uint32_t)(krow_bytes >> 4);
  const bool kfix = (long long)(key_hi - key_lo + 2 * kTK) * krec < (1LL << 31);
  const __amdgpu_buffer_rsrc_t rk = dma_rsrc(kseq + (size_t)key_lo * krow_bytes);
  // K rows of chunk ch into slot buf; rows past the sequence end repeat its
  // last key (they are always masked)
  auto load_k = [&](int ch, int buf) {
    const int kp0 = key_lo + ch * kTK;
    char* kl = smem + buf * BUF;
    if (kp0 + kTK <= seq_len && kfix) {
      const uint32_t u0 = (uint32_t)(ch * kTK) * krec + (koff0 >> 4);
#pragma unroll
      for (int i = 0; i < KIW; ++i) {
        const int j = w + kWaves * i;
        if (NKI % kWaves == 0 || j < NKI)
          lds_dma16(rk, u0 + (uint32_t)(i * KROWS_I) * krec, kl + j * 1024);
      }
      return;
    }
    const char* kb = kseq + (size_t)kp0 * krow_bytes;
    if (kp0 + kTK <= seq_len) {
#pragma unroll
      for (int i = 0; i < KIW; ++i) {
        const int j = w + kWaves * i;
        if (NKI % kWaves == 0 || j < NKI)
          lds_dma16(kb + (size_t)i * KROWS_I * krow_bytes, koff0 >> 4, kl + j * 1024);
      }
    } else {
#pragma unroll
      for (int i = 0; i < KIW; ++i) {
        const int j = w + kWaves * i;
        const int over = max(0, kp0 + krow0 + i * KROWS_I - (seq_len - 1));
        if (NKI % kWaves == 0 || j < NKI)
          lds_dma16(kb, (uint32_t)(((size_t)(i * KROWS_I - over) * krow_bytes + koff0) >> 4),
                    kl + j * 1024);
      }
    }
  };
  // V^T columns of the next chunk in order (staged per block: block gb_next,
  // key offset off_next inside it)
  int gb_next = gb_base + key_lo / a.block_size;
  int off_next = key_lo % a.block_size;
  // Historical and own-block tiles read V^T of one block: one descriptor
  // at the tile's first key, chunk c at record offset 8 c (64 keys of 2
  // bytes); dense tiles cross blocks and address each chunk's block.
  const __amdgpu_buffer_rsrc_t rv = dma_rsrc(
      a.vt + ((size_t)min(gb_next, a.NB - 1) * a.H + h) * D * (size_t)a.block_size + off_next);
  const uint32_t vrow_rec = (uint32_t)(VROWS_I * a.block_size / 8);  // records per instruction step
  uint32_t vch = 0;  // chunks loaded so far
  auto load_v = [&](int buf) {
    char* vl = smem + buf * BUF + KBYTES;
    if (MODE != kModeDense) {
      const uint32_t u0 = vch * (kTK * 2 / 16) + (voff0 >> 4);
#pragma unroll
      for (int i = 0; i < VIW; ++i) {
        const int j = w + kWaves * i;
        if (NVI % kWaves == 0 || j < NVI) lds_dma16(rv, u0 + (uint32_t)i * vrow_rec, vl + j * 1024);
      }
      ++vch;
      return;
    }
    const int gb = min(gb_next, a.NB - 1);
    const char* vb = (const char*)(a.vt + ((size_t)gb * a.H + h) * D * (size_t)a.block_size + off_next);
#pragma unroll
    for (int i = 0; i < VIW; ++i) {
      const int j = w + kWaves * i;
      if (NVI % kWaves == 0 || j < NVI)
        lds_dma16(vb + (size_t)i * VROWS_I * a.block_size * 2, voff0 >> 4, vl + j * 1024);
    }
    off_next += kTK;
    if (off_next == a.block_size) { off_next = 0; ++gb_next; }
  };

  // ---------------- LDS operand addresses ----------------
  // K fragment (row 32 sc + l32, dims 16 ks + 8 hf) sits at segment
  // (2 ks + hf) ^ swz(l32) of its row, i.e. at kbase0 ^ (ks << 5); V^T fragment
  // (row 32 dt + l32, keys 32 sc + 16 mm + 8 hf) at vbase0 ^ ((2 sc + mm) << 5)
  // + dt * 32 rows.  The per-step XOR is recomputed at each use (one VALU op)
  // rather than holding twelve address registers.
  const uint32_t kbase0 = (uint32_t)(l32 * KRB + ((hf ^ swz<KRB>(l32)) << 4));
  const uint32_t vbase0 = (uint32_t)(KBYTES + l32 * VRB + ((hf ^ swz<VRB>(l32)) << 4));
  auto kfrag = [&](uint32_t kb, int slot, int sc, int ks) {
    return *reinterpret_cast<const bf16x8*>(smem + slot * BUF + sc * 32 * KRB + (kb ^ (ks << 5)));
  };
  auto vfrag = [&](uint32_t vb, int slot, int j, int dt) {
    return *reinterpret_cast<const f16x8*>(smem + slot * BUF + dt * 32 * VRB + (vb ^ (j << 5)));
  };

  // ---------------- main loop ----------------
  f32x16 O[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) O[dt][r] = 0.f;
  float m_use = -INFINITY, l_run = 0.f;
  const float scale2 = a.scale2;

  // S[r] is the score of query column (lane & 31) with key kp + 8 (r / 4) + 4 hf + (r % 4)
  auto mask = [&](f32x16& S, int kp) {
    if (!HIST && kp + 31 > wq_min) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (kp + 8 * (r >> 2) + 4 * hf + (r & 3) > qpos) S[r] = -INFINITY;
    }
  };
  auto qk = [&](uint32_t kb, int slot, int sc) {
    f32x16 S;
#pragma unroll
    for (int r = 0; r < 16; ++r) S[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfrag(kb, slot, sc, ks), qreg[ks], S, 0, 0, 0);
    return S;
  };
  // keeps the fragment bases from being hoisted and expanded into one
  // register per step
  auto opaque = [](uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
  };

  // Software pipeline over 64-key chunks, scheduled by hand: in-order issue
  // means a VALU instruction placed between two MFMAs runs while the first
  // is in the matrix pipe, so each MFMA below is followed by a slice of the
  // softmax arithmetic, and by the LDS read of the operand three MFMAs
  // ahead; sched_barrier fences keep the compiler from regrouping them.
  //   A: QK^T(c + 1, keys 0-31)  with  t = s * scale * log2(e) - base and the
  //      row max of chunk c (base: the running max before this chunk);
  //   rescale (rare: the max grew by more than kRescaleSlack);
  //   B: QK^T(c + 1, keys 32-63) with  exp2 of t for keys 0-31,
  //      PV(c, keys 0-31)        with  exp2 of t for keys 32-63,
  //      PV(c, keys 32-63).
  // K and V^T have separate double buffers (slot = chunk parity): iteration
  // c reads K(c + 1) and V(c) and fills K(c + 2) and V(c + 1).
  constexpr int NPV = DT * 2;       // MFMAs of one 32-key PV step
  constexpr int PF = 3;             // LDS operand prefetch distance (MFMAs)
  constexpr int EA = 32 / KS;       // scores scaled per MFMA in A
  constexpr int EB = 16 / KS;       // probabilities per MFMA in QK part of B
  constexpr int EP = 16 / NPV;      // probabilities per MFMA in PV part of B
  static_assert(KS >= PF && NPV >= PF, "prefetch distance");
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
  // probabilities e = exp2(t) of values [v0, v0 + n) of T: rounded to fp16
  // into P, summed in fp32 into l_run
  auto probs_part = [&](const f32x16& T, f16x8* P, int v0, int n) {
#pragma unroll
    for (int v = v0; v < v0 + n; v += 2) {
      const float e0 = __builtin_amdgcn_exp2f(T[v]);
      const float e1 = __builtin_amdgcn_exp2f(T[v + 1]);
      P[v >> 3][v & 7] = (_Float16)e0;
      P[v >> 3][(v + 1) & 7] = (_Float16)e1;
      l_run += e0 + e1;
    }
  };
  auto iteration = [&](int c, f32x16& S0, f32x16& S1, f32x16& N0, f32x16& N1, auto odd_t,
                       auto more_t) {
    // slots of chunks c and c + 1: their parity in the double buffers; in
    // resident tiles chunk c sits at c * BUF, added to the operand bases
    constexpr int CS = (RES || RING4) ? 0 : (decltype(odd_t)::value ? 1 : 0);
    constexpr int NS = (RES || RING4) ? 0 : CS ^ 1;
    constexpr bool MORE = decltype(more_t)::value;
    const uint32_t kshift = RES     ? (uint32_t)((c + 1) * BUF)
                            : RING4 ? (uint32_t)(((c + 1) & 3) * BUF)
                                    : 0u;
    const uint32_t vshift = RES ? (uint32_t)(c * BUF) : RING4 ? (uint32_t)((c & 3) * BUF) : 0u;
    const int kp0 = key_lo + c * kTK;
    mask(S0, kp0);
    mask(S1, kp0 + 32);
    if (RING4) {
      if (c + 3 < nchunks) load_k(c + 3, (c + 3) & 3);
      if (c + 2 < nchunks) load_v((c + 2) & 3);
    }
    const uint32_t kb = opaque(kbase0) + kshift;
    const uint32_t vb = opaque(vbase0) + vshift;
    const float base_old = m_use == -INFINITY ? 0.f : m_use;
    bf16x8 kf[KS], kg[KS];
    f16x8 vf[NPV], vg[NPV];
    auto vread = [&](f16x8* dst, int sc, int i) {
      dst[i] = vfrag(vb, CS, 2 * sc + i / DT, i % DT);
    };
    // ---- A
    float mx = -INFINITY;
    if (MORE) {
#pragma unroll
      for (int ks = 0; ks < PF; ++ks) kf[ks] = kfrag(kb, NS, 0, ks);
#pragma unroll
      for (int r = 0; r < 16; ++r) N0[r] = 0.f;
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      fence();
      if (MORE) {
        N0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qreg[ks], N0, 0, 0, 0);
        if (ks + PF < KS) kf[ks + PF] = kfrag(kb, NS, 0, ks + PF);
        else kg[ks + PF - KS] = kfrag(kb, NS, 1, ks + PF - KS);
      }
#pragma unroll
      for (int v = ks * EA; v < (ks + 1) * EA; v += 2) {
        f32x16& T = v < 16 ? S0 : S1;
        const int r = v & 15;
        T[r] = fmaf(T[r], scale2, -base_old);
        T[r + 1] = fmaf(T[r + 1], scale2, -base_old);
        mx = __builtin_fmaxf(mx, __builtin_fmaxf(T[r], T[r + 1]));
      }
    }
    fence();
    const float cand = max_with_partner(mx);  // in units of t: max(s) * scale2 - base_old
    // per query column: a column's base moves only on its own scores, so its
    // result does not depend on which other queries share the wave
    if (cand > (m_use == -INFINITY ? -INFINITY : kRescaleSlack)) {
      const float m_new = fmaxf(m_use, base_old + cand);
      const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_use - m_new);
      const float delta = (m_new == -INFINITY ? 0.f : m_new) - base_old;
      m_use = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[dt][r] *= alpha;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        S0[r] -= delta;
        S1[r] -= delta;
      }
    }
    // the next chunks' loads go out after the A part, not at the iteration
    // start where every wave of the workgroup issues its operand reads at
    // once after the barrier (1M historical kernel 2% faster, bit-identical)
    if (!RES && !RING4) {
      if (c + 2 < nchunks) load_k(c + 2, CS);
      if (MORE) load_v(NS);
    }
    // ---- B
    const uint32_t kb2 = opaque(kbase0) + kshift;
    f16x8 P0[2], P1[2];
    if (MORE) {
#pragma unroll
      for (int r = 0; r < 16; ++r) N1[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        fence();
        N1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kg[ks], qreg[ks], N1, 0, 0, 0);
        if (ks + PF < KS) kg[ks + PF] = kfrag(kb2, NS, 1, ks + PF);
        else vread(vf, 0, ks + PF - KS);
        probs_part(S0, P0, ks * EB, EB);
      }
    } else {
#pragma unroll
      for (int i = 0; i < PF; ++i) vread(vf, 0, i);
      probs_part(S0, P0, 0, 16);
    }
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      fence();
      O[i % DT] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[i], P0[i / DT], O[i % DT], 0, 0, 0);
      if (i + PF < NPV) vread(vf, 0, i + PF);
      else vread(vg, 1, i + PF - NPV);
      probs_part(S1, P1, i * EP, EP);
    }
#pragma unroll
    for (int i = 0; i < NPV; ++i) {
      fence();
      O[i % DT] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vg[i], P1[i / DT], O[i % DT], 0, 0, 0);
      if (i + PF < NPV) vread(vg, 1, i + PF);
    }
    fence();
  };
  // Output rows (fp16 partials, or bf16 dense output) leave through the
  // wave's LDS staging tile, 64 dims at a time, so that eight lanes store one
  // whole 128-byte line of a row: the accumulator layout gives a lane only
  // 8 bytes of each of its row's lines, and a row would otherwise cost
  // sixteen 16-byte pieces instead of two line writes.  dst[i] is row
  // (lane >> 3) + 8 i of the wave's 32 query columns, already offset by this
  // lane's 16-byte segment (lane & 7); CHECKED: null for rows not stored.
  // The stores are non-temporal: the rows are read once, by a later kernel,
  // and keep the L2 for the K/V chunks (32K: historical 4.15 -> 4.05 ms,
  // own block 0.254 -> 0.215 ms).
  auto stage_out = [&](float inv, char* const* dst, auto checked_t) {
    constexpr bool CHECKED = decltype(checked_t)::value;
    const int ln = (int)opaque((uint32_t)lane);
    const int row = ln & 31, half = ln >> 5;
    char* stg = smem + kStageOff + w * kStageBytes;
#pragma unroll
    for (int dp = 0; dp < DT / 2; ++dp) {
#pragma unroll
      for (int dl = 0; dl < 2; ++dl)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& Od = O[2 * dp + dl];
          const float x0 = Od[4 * g] * inv, x1 = Od[4 * g + 1] * inv;
          const float x2 = Od[4 * g + 2] * inv, x3 = Od[4 * g + 3] * inv;
          u32x2 v2;
          if (MODE == kModeDense) v2 = u32x2{pack_bf16x2(x0, x1), pack_bf16x2(x2, x3)};
          else v2 = u32x2{pack_f16x2(x0, x1), pack_f16x2(x2, x3)};
          *reinterpret_cast<u32x2*>(stg + row * 128 + (((dl * 4 + g) ^ (row & 7)) << 4) +
                                    8 * half) = v2;
        }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = (ln >> 3) + 8 * i;
        const u32x4 d4 =
            *reinterpret_cast<const u32x4*>(stg + r * 128 + (((ln & 7) ^ (r & 7)) << 4));
        if (!CHECKED || dst[i] != nullptr)
          __builtin_nontemporal_store(d4, reinterpret_cast<u32x4*>(dst[i] + dp * 128));
      }
    }
  };
  using yes = std::integral_constant<bool, true>;
  using no = std::integral_constant<bool, false>;
  if constexpr (!RES) {
    if constexpr (RING4) {
      load_k(0, 0);
      load_v(0);
      if (nchunks > 1) {
        load_k(1, 1);
        load_v(1);
      }
      if (nchunks > 2) load_k(2, 2);
      __syncthreads();
      f32x16 S0 = qk(kbase0, 0, 0);
      f32x16 S1 = qk(kbase0, 0, 1);
      f32x16 N0, N1;
      __syncthreads();  // K(0) is read: its slot takes K(4)
      int c = 0;
      // between two barriers, chunks c and c + 1 read K(c + 1), K(c + 2),
      // V(c), V(c + 1) (loaded before the last barrier) and fill K(c + 3),
      // K(c + 4), V(c + 2), V(c + 3): four slots, none read and filled at once
      for (; c + 2 < nchunks; c += 2) {
        iteration(c, S0, S1, N0, N1, no(), yes());
        iteration(c + 1, N0, N1, S0, S1, yes(), yes());
        __syncthreads();
      }
      if (c + 1 < nchunks) {
        iteration(c, S0, S1, N0, N1, no(), yes());
        iteration(c + 1, N0, N1, S0, S1, yes(), no());
      } else {
        iteration(c, S0, S1, N0, N1, no(), no());
      }
    } else {
      load_k(0, 0);
      load_v(0);
      if (nchunks > 1) load_k(1, 1);
      __syncthreads();
      f32x16 S0 = qk(kbase0, 0, 0);
      f32x16 S1 = qk(kbase0, 0, 1);
      f32x16 N0, N1;
      __syncthreads();  // K(0) is read: its slot takes K(2)
      int c = 0;
      for (; c + 2 < nchunks; c += 2) {
        iteration(c, S0, S1, N0, N1, no(), yes());
        __syncthreads();  // K(c + 2) and V(c + 1) have landed; K(c + 1) and V(c) are read
        iteration(c + 1, N0, N1, S0, S1, yes(), yes());
        __syncthreads();
      }
      if (c + 1 < nchunks) {
        iteration(c, S0, S1, N0, N1, no(), yes());
        __syncthreads();
        iteration(c + 1, N0, N1, S0, S1, yes(), no());
      } else {
        iteration(c, S0, S1, N0, N1, no(), no());
      }
    }

    // ---------------- epilogue ----------------
    float out_scale = 1.f;
    if (MODE == kModeDense) out_scale = __builtin_ldexpf(1.0f, v_exponent(a.vmax_bits[h]));
    const float l_tot = sum_with_partner(l_run);
    const float inv = out_scale / l_tot;
    const float lse_val = (m_use + log2f(l_tot)) * kLn2;
    // O[dt][r] is output dim 32 dt + 8 (r / 4) + 4 hf + (r % 4)
    if (MODE != kModeDense || OUT_BF16) {
      // 2-byte rows go out through the staging tile; every lane takes part
      // (columns without a query stage values that are never stored)
      char* dst[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = (lane >> 3) + 8 * i;
        const int lo = __shfl((int)(uint32_t)oidx, r);
        const int hi = __shfl((int)(oidx >> 32), r);
        const long long orow = ((long long)hi << 32) | (uint32_t)lo;
        dst[i] = __shfl(qtok, r) >= 0 ? (char*)a.o_out + orow * (D * 2) + (lane & 7) * 16
                                      : nullptr;
      }
      stage_out(inv, dst, yes());
      if (qtok >= 0 && hf == 0) a.lse_out[oidx] = lse_val;
      return;
    }
    if (qtok < 0) return;  // both lanes of a query column take the same branch
    {
      float* op = (float*)a.o_out + (size_t)oidx * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 v4 = {O[dt][4 * g] * inv, O[dt][4 * g + 1] * inv, O[dt][4 * g + 2] * inv,
                      O[dt][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(op + 32 * dt + 8 * g + 4 * hf) = v4;
        }
    }
    if (hf == 0) a.lse_out[oidx] = lse_val;
  } else {
    // ---------------- resident passes ----------------
    // the whole block once, chunk ch in slot ch; LDS is read-only afterwards,
    // so each wave runs its passes of 32 gathered queries without barriers.
    // A pass's list entries are read one pass ahead, and its queries are
    // gathered at the end of the previous pass, ahead of that pass's output
    // stores (the vector-memory counter is in order), so the gather overlaps
    // the epilogue and does not wait for the stores to be acknowledged; the
    // query registers are free there.  Lanes past the tile's end take the
    // entry of the pass's first row: they compute that query again, bit for
    // bit, and store the same values to the same place, so no store or load
    // needs a branch.
    auto entry = [&](int r, int ln32) {
      const int j = r + ln32 < ti.z ? r + ln32 : min(r, ti.z - 1);
      return a.list[j];
    };
    auto gather = [&](int ent) {
      const int tok = (int)__umulhi((uint32_t)ent, a.topk_magic);  // ent / topk, or one less
      const int tq = ent - tok * a.topk >= a.topk ? tok + 1 : tok;
      const int ln = (int)opaque((uint32_t)lane);
      const uint16_t* qp = a.q + ((size_t)tq * a.Hs + hg) * D + 8 * (ln >> 5);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qreg[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 16 * ks));
    };
    for (int ch = 0; ch < nchunks; ++ch) {
      load_k(ch, ch);
      load_v(ch);
    }
    int r0 = ti.y + w * 32;
    int ent = entry(r0, l32);
    gather(ent);
    // the first pass's queries have landed before the loop: inside it, the
    // query registers then only ever wait for the gather issued one pass
    // earlier, never for the output stores queued behind it
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(qreg[ks]));
    __syncthreads();
    f32x16 S0, S1, N0, N1;
    for (; r0 < ti.z; r0 += kWaves * 32) {
      const int ent_next = entry(r0 + kWaves * 32, (int)opaque((uint32_t)lane) & 31);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) O[dt][r] = 0.f;
      m_use = -INFINITY;
      l_run = 0.f;
      {
        const uint32_t kb0 = opaque(kbase0);
        S0 = qk(kb0, 0, 0);
        S1 = qk(kb0, 0, 1);
      }
      int c = 0;
      for (; c + 2 < nchunks; c += 2) {
        iteration(c, S0, S1, N0, N1, no(), yes());
        iteration(c + 1, N0, N1, S0, S1, yes(), yes());
      }
      if (c + 1 < nchunks) {
        iteration(c, S0, S1, N0, N1, no(), yes());
        iteration(c + 1, N0, N1, S0, S1, yes(), no());
      } else {
        iteration(c, S0, S1, N0, N1, no(), no());
      }
      gather(ent_next);
      // fp16 partial (V units) and lse of the pass's rows
      {
        auto out_row = [&](int e) {  // partial row of list entry e
          int qt = (int)__umulhi((uint32_t)e, a.topk_magic);  // e / topk, or one less
          int slot = e - qt * a.topk;
          if (slot >= a.topk) { ++qt; slot -= a.topk; }
          return ((long long)qt * a.H + h) * a.topk + slot;
        };
        const float l_tot = sum_with_partner(l_run);
        const int ln = (int)opaque((uint32_t)lane);
        const long long orow = out_row(ent);
        a.lse_out[orow] = (m_use + log2f(l_tot)) * kLn2;  // both lanes: same value
        char* dst[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = (ln >> 3) + 8 * i;
          const int lo = __shfl((int)(uint32_t)orow, r);
          const int hi = __shfl((int)(orow >> 32), r);
          dst[i] = (char*)a.o_out + (((long long)hi << 32) | (uint32_t)lo) * (D * 2) + (ln & 7) * 16;
        }
        stage_out(1.f / l_tot, dst, no());
      }
      ent = ent_next;
    }
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
  a.H = g.head_cnt;
  a.Hs = g.num_heads;
  a.h0 = g.head_lo;
  a.block_size = g.block_size;
  a.topk = topk;
  a.NB = g.total_blocks;
  a.scale2 = scale * kLog2e;
  a.topk_magic = 0xFFFFFFFFu / (uint32_t)topk;
  a.q_limit = 0x7fffffff;
  return a;
}

template <int D, int MODE, bool OB>
static void launch_mfma(int waves, dim3 grid, hipStream_t st, const MfmaArgs& a) {
  if (waves == 8)
    hipLaunchKernelGGL((attn_mfma_kernel<D, MODE, OB, 8>), grid, dim3(64 * 8), 0, st, a);
  else
    hipLaunchKernelGGL((attn_mfma_kernel<D, MODE, OB, 4>), grid, dim3(64 * 4), 0, st, a);
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
  // tile_info was cut into tiles of hist_tile_q(block_size, head_dim) queries
  dim3 grid((unsigned)max_tiles);
  if (hist_resident(g.block_size, g.head_dim)) {
    if (g.head_dim == 128)
      hipLaunchKernelGGL((attn_mfma_kernel<128, kModeHistRes, true, 8>), grid, dim3(64 * 8), 0,
                         st, a);
    else
      hipLaunchKernelGGL((attn_mfma_kernel<64, kModeHistRes, true, 8>), grid, dim3(64 * 8), 0,
                         st, a);
    return hipGetLastError();
  }
  const int waves = mfma_waves(g.block_size);
  if (g.head_dim == 128) launch_mfma<128, kModeHist, true>(waves, grid, st, a);
  else launch_mfma<64, kModeHist, true>(waves, grid, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_mfma_own(const void* q, const void* k, const uint16_t* vt,
                                const Geo& g, int topk, float scale, uint16_t* o_part,
                                float* lse_part, int dense_blocks, const int32_t* notfull,
                                hipStream_t st) {
  if (g.total_tokens == 0 || g.max_seqlen == 0) return hipSuccess;
  MfmaArgs a = base_args(q, k, vt, g, topk, scale);
  a.dense_blocks = dense_blocks;
  a.notfull = notfull;
  // own-block tiles span at most one block of keys: 4 waves
  const int waves = 4;
  a.tiles_per_unit = (g.block_size + 32 * waves - 1) / (32 * waves);
  a.units_per_seq = (g.max_seqlen + g.block_size - 1) / g.block_size;
  a.o_out = o_part;
  a.lse_out = lse_part;
  dim3 grid((unsigned)(g.num_seqs * a.tiles_per_unit * a.units_per_seq), g.head_cnt);
  if (g.head_dim == 128) launch_mfma<128, kModeOwn, true>(waves, grid, st, a);
  else launch_mfma<64, kModeOwn, true>(waves, grid, st, a);
  return hipGetLastError();
}

hipError_t launch_attn_mfma_dense(const void* q, const void* k, const uint16_t* vt,
                                  const uint32_t* vmax_bits, const Geo& g, float scale,
                                  void* out, bool out_bf16, float* lse, hipStream_t st,
                                  int q_limit) {
  if (g.total_tokens == 0 || g.max_seqlen == 0 || q_limit <= 0) return hipSuccess;
  MfmaArgs a = base_args(q, k, vt, g, 1, scale);
  a.vmax_bits = vmax_bits;
  a.q_limit = q_limit;
  const int span = min(g.max_seqlen, q_limit);  // query positions of the longest sequence
  const int waves = mfma_waves(span);
  a.tiles_per_unit = (span + 32 * waves - 1) / (32 * waves);  // dense_grid's tiles
  a.units_per_seq = 1;
  a.o_out = out;
  a.lse_out = lse;
  dim3 grid((unsigned)(g.num_seqs * a.tiles_per_unit), g.head_cnt);
  if (g.head_dim == 128) {
    if (out_bf16) launch_mfma<128, kModeDense, true>(waves, grid, st, a);
    else launch_mfma<128, kModeDense, false>(waves, grid, st, a);
  } else {
    if (out_bf16) launch_mfma<64, kModeDense, true>(waves, grid, st, a);
    else launch_mfma<64, kModeDense, false>(waves, grid, st, a);
  }
  return hipGetLastError();
}

}  // namespace moba
