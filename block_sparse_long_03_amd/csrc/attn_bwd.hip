// Backward of the MoBA block attention on gfx950: bf16 MFMA, fp32 accumulation.
//
// The block selection is a hard top-k and is not differentiated ("MoBA:
// Learned Block Sparsity for Long-Context Attention", "The Change"; the
// elamur.ai summary, "Key points": trained end to end with the gate's
// choice held fixed); gradients reach q, K and V through the softmax
// attention over each query's selected tokens.  With P = exp(scale q.k - lse)
// (lse from the forward pass, so P is the final softmax weight of the pair),
// Dq = dO_q . O_q and dP = dO_q . v_k:
//   dV_k += P dO_q,   dS = P (dP - Dq),   dK_k += scale dS q,   dQ_q += scale dS k
//
// Three kernels:
//   bwd_prep:  Dq = rowsum(dO * O) per (token, head) and dq = 0.
//   bwd_kv:    KV-centric.  A workgroup owns 128 keys of one (head, KV
//              block), 32 per pair of waves, and streams every query that
//              attends them: the block's historical list (queries that
//              selected it), then the own-block queries at or after its
//              first key (causal mask).  dK and dV stay in registers for the
//              whole stream and are written once: no atomics (the sums
//              follow the list order, which depends on scheduling).
//   bwd_q:     the forward's tiles (a (head, block) list tile of gathered
//              queries, or an own-block query tile) against the block's keys
//              in 64-key chunks; each wave keeps its 32 queries' dQ in
//              registers and adds it to the fp32 dq once per tile with
//              coalesced atomics (a query gets at most topk additions).
//
// Products:
//   bwd_kv:  S = Q K^T and dP = dO V^T (A = query rows from LDS, B = a
//            wave's key rows in registers), then dV^T += dO^T P and
//            dK^T += Q^T dS, whose A operands (dims x queries) come from the
//            row-major query tiles through the LDS transpose read
//            (ds_read_b64_tr_b16).
//   bwd_q:   S^T = K Q^T and dP^T = V dO^T (A = key rows from LDS, B = the
//            wave's query rows in registers), then dQ^T += K^T dS^T with K^T
//            again from the transpose read.
// In both, the C layout of the first products (lane = one column, 16 rows
// in the MFMA row order 8(r/4) + 4(lane/32) + r%4) is used as the B operand
// of the last ones directly: the A operand's k index follows the same order,
// which the transpose read produces by picking the rows it gathers.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace moba {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

enum { kBwdHist = 0, kBwdOwn = 1 };

constexpr int kBwdWaves = 4;
constexpr int kBwdKeysPerWave = 32;
constexpr int kBwdKeysPerWg = 4 * kBwdKeysPerWave;  // bwd_kv: 4 wave pairs x 32 keys
constexpr int kBwdQTile = 64;                               // queries per bwd_kv step
constexpr int kBwdChunk = 64;                               // keys per bwd_q step

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* dout;
  const float* lse;   // [T, H] natural log, from the forward pass
  const float* dvec;  // [T, H] rowsum(dO * O)
  const int32_t* cu_seqlens;
  const int32_t* cu_blocks;
  int num_seqs, total_tokens, H, block_size, topk, NB;
  int tiles_per_unit;  // bwd_q own: query tiles per block
  int units_per_seq;   // bwd_q own: max blocks per sequence
  int kgroups;         // bwd_kv: key groups per block (block_size / 128)
  float scale, scale2;  // softmax scale, scale * log2(e)
  const int32_t* list;     // per (head, block) list of the global tokens that selected it
  const int32_t* offsets;  // list range of key h * NB + gb
  const int4* tile_info;   // bwd_q historical tiles
  float* dq;
  float* dk;
  float* dv;
};

// 16-byte segment swizzle of a tile row: rows of 256 B (d = 128) or 128 B
// (d = 64), 64 banks of 4 bytes.  A 16-lane pass of operand row reads (16
// consecutive rows, one segment each) and a 32-lane pass of the transpose
// read (4 consecutive rows x 4 consecutive segments) both hit distinct banks:
// the 4 rows of a transpose pass land in different quarters of the banks.
template <int ROWB>
__device__ __forceinline__ int bswz(int row) {
  if (ROWB == 256) return 4 * (row & 3) + ((row >> 2) & 3);
  const int m = (row >> 1) & 7;
  return 4 * (m & 1) + ((m >> 1) & 3);
}


// 16 bytes per lane from a per-lane global address into LDS (dst + 16 lane).
// The rows of a query-list tile are arbitrary tokens, whose offsets from any
// one base can exceed the 32-bit reach of the buffer form; this form takes a
// full address per lane, at the price of coarser LDS waits while it is in
// flight (see lds_dma16).
typedef __attribute__((address_space(3))) void lds_flat_t;
__device__ __forceinline__ void lds_dma16_flat(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_flat_t*)dst, 16, 0, 0);
}

// A operand X^T (dims 32 dt .. + 31 as rows, 16 tile rows R0 .. R0 + 15 as k)
// from a row-major bf16 tile X: the k order is the MFMA output row order, so
// it pairs with a B operand taken from an MFMA result's registers 8 s .. 8 s + 7.
// off[0] / off[1] are the lane's byte offsets of its two 8-byte reads
// relative to row R0 (a multiple of 16).
//
// The reads go through a restrict-qualified pointer.  The alias scope that
// gives the read lets the compiler's wait insertion treat it like any other
// LDS load; without it, every transpose read waits for all of the wave's LDS
// DMA still in flight, i.e. for the prefetch of a later tile.  The kernels
// order DMA and reads themselves: a tile is read only after the barrier that
// follows the vmcnt(0) wait of the iteration that issued it.
__device__ __forceinline__ s16x4 ds_read_tr(const lds_s16x4* __restrict__ p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}
__device__ __forceinline__ bf16x8 tr_frag(const char* tile_r0, uint32_t off0, uint32_t off1) {
  const s16x4 a = ds_read_tr((const lds_s16x4*)(tile_r0 + off0));
  const s16x4 b = ds_read_tr((const lds_s16x4*)(tile_r0 + off1));
  const s16x8 c = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, c);
}

// the lane's two transpose-read offsets for dims 32 dt .. 32 dt + 31: lane
// l of group g = l / 16 (index i = l % 16) points at row 4 (g / 2) + i / 4
// (+ 8 for the second read) and dims 32 dt + 16 (g % 2) + 4 (i % 4) .. + 3;
// the read hands lane l the four values of dim 32 dt + l % 32 at rows
// 4 (l / 32) + 0..3 (resp. 8 + ...), i.e. k = 8 (l / 32) + 0..7 in MFMA order.
template <int ROWB>
__device__ __forceinline__ uint32_t tr_offset(int lane, int dt, int second) {
  const int g = lane >> 4, i = lane & 15;
  const int row = 4 * (g >> 1) + (i >> 2) + 8 * second;
  const int col_b = 2 * (32 * dt + 16 * (g & 1) + 4 * (i & 3));
  const int seg = col_b >> 4;
  return (uint32_t)(row * ROWB + ((seg ^ bswz<ROWB>(row)) << 4) + (col_b & 15));
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) { return pack_bf16x2(lo, hi); }

// acc += A B with the accumulator pinned to AGPRs.  The dK^T / dV^T sums of
// the key-centric kernel live there for the whole query stream, which leaves
// the VGPRs to the stream's operands and scores; left to the register
// allocator, the two register files trade whole 16-register accumulators
// every step.  The compiler sees an opaque instruction here, so the MFMA
// hazards are covered by hand: `settle` (issued before the accumulators are
// read by anything else) waits out the last MFMA's write, and the VGPR
// operands written by VALU code are five wait states old when first read.
__device__ __forceinline__ void mfma_acc_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc_agpr_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void zero_agpr(f32x16& acc) {
  const bf16x8 z = {};
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc) : "v"(z));
}
__device__ __forceinline__ void settle(f32x16& acc) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(acc));
}

// bf16 B fragment from registers 8 s .. 8 s + 7 of an fp32 MFMA result
__device__ __forceinline__ bf16x8 regs_to_bf16(const f32x16& x, int s) {
  u32x4 w;
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = pack_bf16(x[8 * s + 2 * i], x[8 * s + 2 * i + 1]);
  return __builtin_bit_cast(bf16x8, w);
}

// ---------------------------------------------------------------------------
// prep: Dq = rowsum(dO * O) (fp32), lse log2(e) for bwd_kv, and dq = 0
// ---------------------------------------------------------------------------
template <int D, bool OUT_F32>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const void* __restrict__ out,
                                                       const uint16_t* __restrict__ dout,
                                                       const float* __restrict__ lse,
                                                       long long rows, float* __restrict__ dvec,
                                                       float* __restrict__ lse2,
                                                       float* __restrict__ dq) {
  constexpr int PER = D / 16;  // elements per lane (16 lanes per row)
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int li = threadIdx.x & 15;
  float acc = 0.f;
  if (row < rows) {
    const size_t base = (size_t)row * D + li * PER;
    float o[PER], g[PER];
    if constexpr (OUT_F32) {
#pragma unroll
      for (int e = 0; e < PER; e += 4) {
        const f32x4 x = *reinterpret_cast<const f32x4*>((const float*)out + base + e);
#pragma unroll
        for (int u = 0; u < 4; ++u) o[e + u] = x[u];
      }
    } else {
#pragma unroll
      for (int e = 0; e < PER; e += 2) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>((const uint16_t*)out + base + e);
        o[e] = lo_bf16(w);
        o[e + 1] = hi_bf16(w);
      }
    }
#pragma unroll
    for (int e = 0; e < PER; e += 2) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(dout + base + e);
      g[e] = lo_bf16(w);
      g[e + 1] = hi_bf16(w);
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) acc = fmaf(o[e], g[e], acc);
#pragma unroll
    for (int e = 0; e < PER; e += 4)
      *reinterpret_cast<f32x4*>(dq + base + e) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
  if (row < rows && li == 0) {
    dvec[row] = acc;
    lse2[row] = lse[row] * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// bwd_kv, paired waves: dK, dV of 128 keys of one (head, KV block) with 8
// waves.  Waves w and w + 4 share the keys 32 (w % 4) .. + 31 and split the
// work of each 32-query half: wave w (the P wave) forms S = Q K^T, P and
// dV^T += dO^T P; wave w + 4 (the dS wave) forms dP = dO V^T, takes P
// through LDS, and accumulates dK^T += Q^T dS with dS = P (dP - Dq).  Each
// wave holds one key-row operand (K or V) and one 64-register accumulator,
// which brings it to two waves per SIMD; the two waves of a pair sit on one
// SIMD (wave ids w and w + 4), so one's softmax arithmetic runs beside the
// other's products.
// ---------------------------------------------------------------------------
constexpr int kBwdPairWaves = 8;

constexpr int kListSlots = 4;  // list slices of four tiles in LDS

// 4 bytes per lane from a per-lane global address into LDS (dst + 4 lane)
__device__ __forceinline__ void lds_dma4_flat(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_flat_t*)dst, 4, 0, 0);
}

// Workgroup barrier that leaves the wave's newest n vector-memory loads in
// flight (all of them LDS DMA, whose data no wave reads before a later
// barrier) and completes everything older; the LDS accesses of the wave are
// complete too.  n is wave-uniform and at most 8.
__device__ __forceinline__ void tile_barrier(int n) {
  switch (n) {
#define MOBA_TB(N) \
    case N: asm volatile("s_waitcnt vmcnt(" #N ") lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
    MOBA_TB(1) MOBA_TB(2) MOBA_TB(3) MOBA_TB(4) MOBA_TB(5) MOBA_TB(6) MOBA_TB(7) MOBA_TB(8)
#undef MOBA_TB
    default: asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
  }
}

// LDS handoff between the waves of a workgroup: the wave's own LDS accesses
// are complete, then the barrier.  Unlike __syncthreads it does not wait for
// vector memory, so the DMA of later tiles stays in flight; the asm's memory
// clobber keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int D>
__global__ __launch_bounds__(64 * kBwdPairWaves) void bwd_kv_pair_kernel(BwdArgs a) {
  constexpr int KS = D / 16;   // k-steps over dims
  constexpr int DT = D / 32;   // 32-dim tiles
  constexpr int ROWB = D * 2;  // bytes of a query row in LDS
  constexpr int TBYTES = kBwdQTile * ROWB;  // one query tile (Q or dO)
  constexpr int LPR = ROWB / 16;            // lanes per row in a DMA instruction
  constexpr int RPI = 64 / LPR;             // rows per DMA instruction
  constexpr int NI = kBwdQTile / RPI;       // DMA instructions per tile and tensor
  constexpr int NIW = NI / kBwdPairWaves;   // ... per wave
  static_assert(NI % kBwdPairWaves == 0, "whole wave loads");
  constexpr int NBUF = 3;                   // tile slots
  constexpr int SBYTES = 2 * kBwdQTile * 4; // lse and Dq of one tile
  constexpr int XBYTES = 64 * 16 * 4;       // one 32 x 32 fp32 tile of P, C layout
  // LDS: Q ring | dO ring | statistics ring | P exchange | list ring.  Every
  // operand read adds a per-lane register offset (which holds the ring's
  // start) to a compile-time slot and half offset below 64 KiB, which the
  // LDS instruction carries as its immediate: no address arithmetic per read.
  constexpr int Q_OFF = 0;
  constexpr int O_OFF = NBUF * TBYTES;
  constexpr int S_OFF = 2 * NBUF * TBYTES;
  constexpr int X_OFF = S_OFF + NBUF * SBYTES;
  constexpr int L_OFF = X_OFF + 4 * 2 * XBYTES;
  constexpr int LDS_BYTES = L_OFF + kListSlots * kBwdQTile * 4;
  static_assert((NBUF - 1) * TBYTES + 48 * ROWB < 65536, "immediate offsets");
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pw = w & 3;           // pair: keys 32 pw .. of the workgroup
  const bool pwave = w < 4;       // the P wave of the pair (else the dS wave)
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int kg = L % a.kgroups;
  const int bk = L / a.kgroups;  // h * NB + gb
  const int h = bk / a.NB;
  const int gb = bk - h * a.NB;
  const int sq = seq_of_block(a.cu_blocks, a.num_seqs, gb);
  int seq_start, seq_len;
  seq_span(a.cu_seqlens, sq, a.total_tokens, &seq_start, &seq_len);
  const int blo = (gb - a.cu_blocks[sq]) * a.block_size;
  const int bhi = min(blo + a.block_size, seq_len);
  const int kwg = blo + kg * kBwdKeysPerWg;
  if (kwg >= bhi) return;
  const int kw = kwg + pw * kBwdKeysPerWave;
  const int key = kw + l32;
  const bool key_ok = key < bhi;

  // ---- the wave's key rows: K (P wave) or V (dS wave), B operand of its product
  bf16x8 brow[KS];
  {
    const size_t row = ((size_t)seq_start + min(key, bhi - 1)) * a.H + h;
    const uint16_t* bp = (pwave ? a.k : a.v) + row * D + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      brow[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(bp + 16 * ks));
  }

  // ---- the query stream: historical list tiles, then own-block tiles.
  // Everything a tile needs reaches LDS by DMA (list entries, Q and dO rows,
  // lse and Dq), and no register waits on a vector-memory load inside the
  // loop, so the barrier that ends iteration t waits only for what earlier
  // iterations issued: the list slice of tile x is loaded at iteration x - 4,
  // its rows and statistics at iteration x - 2, and it is read at iteration x.
  const int e0 = a.offsets[bk], e1 = a.offsets[bk + 1];
  const int n_hist = (e1 - e0 + kBwdQTile - 1) / kBwdQTile;
  const int own_q0 = kwg;
  const int n_own = (bhi - own_q0 + kBwdQTile - 1) / kBwdQTile;
  const int ntiles = n_hist + n_own;
  const int lseg = lane % LPR;
  int32_t* lring = (int32_t*)(smem + L_OFF);  // kListSlots x 64 entries
  auto rows_of = [&](int t) {  // valid rows of tile t
    return t < n_hist ? min(kBwdQTile, e1 - e0 - t * kBwdQTile)
                      : min(kBwdQTile, bhi - own_q0 - (t - n_hist) * kBwdQTile);
  };
  // global token of row r of tile t (rows past the end repeat the last one)
  auto tile_row = [&](int t, int r) {
    if (t < n_hist) return lring[(t % kListSlots) * kBwdQTile + min(r, rows_of(t) - 1)];
    return seq_start + min(own_q0 + (t - n_hist) * kBwdQTile + r, bhi - 1);
  };
  auto issue_list = [&](int t) {  // wave 1: list entries of historical tile t
    const int j = min(e0 + t * kBwdQTile + lane, e1 - 1);
    lds_dma4_flat(a.list + j, lring + (t % kListSlots) * kBwdQTile);
  };
  auto issue_tile = [&](int t, auto slot_t) {
    constexpr int SLOT = decltype(slot_t)::value;
    char* qd = smem + Q_OFF + SLOT * TBYTES;
    char* od = smem + O_OFF + SLOT * TBYTES;
    if (w == 0) {
      const size_t ri = (size_t)tile_row(t, lane) * a.H + h;
      float* sl = (float*)(smem + S_OFF + SLOT * SBYTES);
      lds_dma4_flat(a.lse + ri, sl);
      lds_dma4_flat(a.dvec + ri, sl + kBwdQTile);
    }
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
      const int j = w + kBwdPairWaves * i;
      const int r = j * RPI + lane / LPR;
      const size_t src = (((size_t)tile_row(t, r) * a.H + h) * D) * 2 + ((lseg ^ bswz<ROWB>(r)) << 4);
      lds_dma16_flat((const char*)a.q + src, qd + j * 1024);
      lds_dma16_flat((const char*)a.dout + src, od + j * 1024);
    }
  };
  // vector-memory instructions this wave issues in iteration t
  auto issued_in = [&](int t) {
    int n = 0;
    if (t + 2 < ntiles) n += 2 * NIW + (w == 0 ? 2 : 0);
    if (w == 1 && t + 4 < n_hist) n += 1;
    return n;
  };

  // ---- per-lane LDS offsets, computed once and kept in registers (the asm
  // keeps the compiler from folding them back into per-read arithmetic)
  auto opaque = [](uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
  };
  const uint32_t rbase = (uint32_t)(l32 * ROWB + ((hf ^ bswz<ROWB>(l32)) << 4));
  uint32_t aoff[KS];  // A rows of S / dP: Q (P wave) or dO (dS wave)
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) aoff[ks] = opaque((pwave ? Q_OFF : O_OFF) + (rbase ^ (ks << 5)));
  uint32_t toff[2][DT];  // transpose reads for dV / dK: dO (P wave) or Q (dS wave)
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    toff[0][dt] = opaque((pwave ? O_OFF : Q_OFF) + tr_offset<ROWB>(lane, dt, 0));
    toff[1][dt] = opaque((pwave ? O_OFF : Q_OFF) + tr_offset<ROWB>(lane, dt, 1));
  }
  const uint32_t soff = opaque(S_OFF + 16 * hf);                      // rows 8 m + 4 hf ..
  const uint32_t xoff = opaque(X_OFF + pw * 2 * XBYTES + 16 * lane);  // P exchange, C layout

  f32x16 acc[DT];  // dV^T (P wave) or dK^T (dS wave)
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) zero_agpr(acc[dt]);

  constexpr int PF = 3;
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
  // P of the pair's current half in C layout: register chunk c of lane l at
  // 16 bytes x (64 c + l), so that each 16-lane pass covers 256 bytes

  auto step = [&](int t, auto slot_t, auto half_t) {
    constexpr int SLOT = decltype(slot_t)::value;
    constexpr int HALF = decltype(half_t)::value;
    constexpr int CA = SLOT * TBYTES + HALF * 32 * ROWB;      // half's rows in its ring
    constexpr int CS = SLOT * SBYTES + HALF * 32 * 4;         // half's lse (Dq: + 256)
    constexpr int CX = HALF * XBYTES;
    // ---- S = Q K^T (P wave) or dP = dO V^T (dS wave)
    bf16x8 af[KS];
#pragma unroll
    for (int i = 0; i < PF; ++i) af[i] = *reinterpret_cast<const bf16x8*>(smem + aoff[i] + CA);
    f32x16 X;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      fence();
      if (ks == 0) {
        const f32x16 z = {};
        X = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[0], brow[0], z, 0, 0, 0);
      } else {
        X = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks], brow[ks], X, 0, 0, 0);
      }
      if (ks + PF < KS) af[ks + PF] = *reinterpret_cast<const bf16x8*>(smem + aoff[ks + PF] + CA);
    }
    fence();
    if (pwave) {
      // P = exp2(S scale log2e - lse log2e) (a.lse holds lse log2e here),
      // the masks, then P to the pair
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(smem + soff + CS + 32 * m);
#pragma unroll
        for (int u = 0; u < 4; ++u)
          X[4 * m + u] = __builtin_amdgcn_exp2f(fmaf(X[4 * m + u], a.scale2, -l4[u]));
      }
      // rows past the tile's end repeat its last row: P = 0 there
      const int vrows = rows_of(t) - 32 * HALF;
      if (vrows < 32) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + 4 * hf + (r & 3) >= vrows) X[r] = 0.f;
      }
      const bool own = t >= n_hist;
      const int qpos0 = own_q0 + (t - n_hist) * kBwdQTile + 32 * HALF;
      if (own && kw + kBwdKeysPerWave - 1 > qpos0) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key > qpos0 + 8 * (r >> 2) + 4 * hf + (r & 3)) X[r] = 0.f;
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<f32x4*>(smem + xoff + CX + 1024 * c) =
            f32x4{X[4 * c], X[4 * c + 1], X[4 * c + 2], X[4 * c + 3]};
    }
    lds_barrier();  // P of this half is in LDS
    if (!pwave) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4 p4 = *reinterpret_cast<const f32x4*>(smem + xoff + CX + 1024 * c);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(smem + soff + CS + 256 + 32 * c);
#pragma unroll
        for (int u = 0; u < 4; ++u) X[4 * c + u] = p4[u] * (X[4 * c + u] - d4[u]);
      }
    }
    // ---- dV^T += dO^T P (P wave) or dK^T += Q^T dS (dS wave)
    bf16x8 xb16[2];
    xb16[0] = regs_to_bf16(X, 0);
    xb16[1] = regs_to_bf16(X, 1);
    constexpr int NB = 2 * DT;  // MFMA i: dt = i / 2, s = i % 2
    auto trf = [&](int i) {
      return tr_frag(smem + CA + (i & 1) * 16 * ROWB, toff[0][i >> 1], toff[1][i >> 1]);
    };
    bf16x8 tf[NB];
#pragma unroll
    for (int i = 0; i < PF; ++i) tf[i] = trf(i);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      fence();
      if (i == 0)
        mfma_acc_agpr_first(acc[0], tf[0], xb16[0]);
      else
        mfma_acc_agpr(acc[i >> 1], tf[i], xb16[i & 1]);
      if (i + PF < NB) tf[i + PF] = trf(i + PF);
    }
    fence();
  };
  using c0 = std::integral_constant<int, 0>;
  using c1 = std::integral_constant<int, 1>;
  using c2 = std::integral_constant<int, 2>;
  // tile t in slot SLOT = t % 3: its two halves, then the barrier
  auto tile = [&](int t, auto slot_t) {
    constexpr int SLOT = decltype(slot_t)::value;
    step(t, slot_t, c0());
    // every wave is past tile t - 1: its slot takes tile t + 2.  The loads
    // go out after the first half, not right after the barrier where every
    // wave reads its first operands
    if (t + 2 < ntiles) issue_tile(t + 2, std::integral_constant<int, (SLOT + 2) % NBUF>());
    if (w == 1 && t + 4 < n_hist) issue_list(t + 4);
    step(t, slot_t, c1());
    // everything issued before this iteration has landed (tile t + 1, the
    // list slice of tile t + 3); this iteration's loads stay in flight
    tile_barrier(issued_in(t));
  };

  if (w == 1)
    for (int x = 0; x < 4 && x < n_hist; ++x) issue_list(x);
  __syncthreads();  // list slices of tiles 0 - 3
  if (ntiles > 0) issue_tile(0, c0());
  if (ntiles > 1) issue_tile(1, c1());
  __syncthreads();  // tiles 0 and 1
  int t = 0;
  for (; t + 3 <= ntiles; t += 3) {
    tile(t, c0());
    tile(t + 1, c1());
    tile(t + 2, c2());
  }
  if (t < ntiles) tile(t, c0());
  if (t + 1 < ntiles) tile(t + 1, c1());

#pragma unroll
  for (int dt = 0; dt < DT; ++dt) settle(acc[dt]);
  if (!key_ok) return;
  const size_t orow = (((size_t)seq_start + key) * a.H + h) * D;
  float* dst = pwave ? a.dv : a.dk;
  const float sc = pwave ? 1.f : a.scale;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int d0 = 32 * dt + 8 * m + 4 * hf;
      *reinterpret_cast<f32x4*>(dst + orow + d0) =
          f32x4{acc[dt][4 * m] * sc, acc[dt][4 * m + 1] * sc, acc[dt][4 * m + 2] * sc,
                acc[dt][4 * m + 3] * sc};
    }
}

// ---------------------------------------------------------------------------
// bwd_q: dQ of one forward tile (4 waves x 32 queries) over its block's keys
// ---------------------------------------------------------------------------
template <int D, int MODE>
__global__ __launch_bounds__(64 * kBwdWaves) void bwd_q_kernel(BwdArgs a) {
  constexpr int KS = D / 16;
  constexpr int DT = D / 32;
  constexpr int ROWB = D * 2;
  constexpr int CBYTES = kBwdChunk * ROWB;  // one K or V chunk
  constexpr int NI = CBYTES / 1024;         // DMA instructions per chunk and tensor
  constexpr int NIW = NI / kBwdWaves;
  constexpr int RPI = 1024 / ROWB;          // rows per DMA instruction
  static_assert(NI % kBwdWaves == 0, "whole wave loads");
  constexpr int BUF = 2 * CBYTES;           // K chunk + V chunk
  constexpr int TQ = kBwdWaves * 32;
  constexpr int TS = D + 4;                 // floats per row of the final dQ staging
  constexpr int SMEM = 2 * BUF > kBwdWaves * 32 * TS * 4 ? 2 * BUF : kBwdWaves * 32 * TS * 4;
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hf = lane >> 5;

  // ---- tile decode (as the forward's historical / own tiles)
  int h, seq_start, seq_len, key_lo, key_hi;
  int qtok = -1, qpos = 0x7fffffff;
  if (MODE == kBwdHist) {
    const int4 ti = a.tile_info[blockIdx.x];
    if (ti.x < 0) return;
    h = ti.x / a.NB;
    const int gb = ti.x - h * a.NB;
    const int s = seq_of_block(a.cu_blocks, a.num_seqs, gb);
    seq_span(a.cu_seqlens, s, a.total_tokens, &seq_start, &seq_len);
    key_lo = (gb - a.cu_blocks[s]) * a.block_size;
    key_hi = min(key_lo + a.block_size, seq_len);
    const int j = ti.y + w * 32 + l32;
    if (j < ti.z) qtok = a.list[j];
  } else {
    const int L = xcd_remap(blockIdx.x + blockIdx.y * gridDim.x, gridDim.x * gridDim.y);
    const int bx = L % gridDim.x;
    h = L / gridDim.x;
    const int per_seq = a.tiles_per_unit * a.units_per_seq;
    const int s = bx / per_seq;
    const int rem = per_seq - 1 - (bx % per_seq);  // heavy tiles first
    seq_span(a.cu_seqlens, s, a.total_tokens, &seq_start, &seq_len);
    const int c = rem / a.tiles_per_unit;
    const int sub = rem % a.tiles_per_unit;
    key_lo = c * a.block_size;
    const int q_lo = key_lo + sub * TQ;
    const int q_hi = min(min(q_lo + TQ, key_lo + a.block_size), seq_len);
    if (q_lo >= q_hi) return;
    key_hi = q_hi;
    const int p = q_lo + w * 32 + l32;
    if (p < q_hi) { qtok = seq_start + p; qpos = p; }
  }
  const bool qv = qtok >= 0;
  const size_t qrow = ((size_t)(qv ? qtok : seq_start) * a.H + h);
  const float lse2 = qv ? a.lse[qrow] * kLog2e : INFINITY;  // invalid query: P = 0
  const float dq_d = qv ? a.dvec[qrow] : 0.f;
  bf16x8 qreg[KS], oreg[KS];
  {
    const uint16_t* qp = a.q + qrow * D + 8 * hf;
    const uint16_t* op = a.dout + qrow * D + 8 * hf;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qreg[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(qp + 16 * ks));
      oreg[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(op + 16 * ks));
    }
  }
  // smallest query position of the wave (own mode: chunks past it need the mask)
  int wq_min = qv ? qpos : 0x7fffffff;
  for (int o = 32; o >= 1; o >>= 1) wq_min = min(wq_min, __shfl_xor(wq_min, o));

  // ---- K and V chunks of 64 keys; rows past the sequence end repeat its
  //      last key (masked)
  const int nchunks = (key_hi - key_lo + kBwdChunk - 1) / kBwdChunk;
  const int lseg = lane % (ROWB / 16);
  auto load_chunk = [&](int ch, int b) {
    char* kd = smem + b * BUF;
    char* vd = kd + CBYTES;
    const int kp0 = key_lo + ch * kBwdChunk;
    const size_t row0 = (((size_t)seq_start + kp0) * a.H + h) * D * 2;
    const char* kbase = (const char*)a.k + row0;
    const char* vbase = (const char*)a.v + row0;
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
      const int j = w + kBwdWaves * i;
      const int r = j * RPI + lane / (ROWB / 16);
      // 16-byte unit of the row's segment relative to the chunk's first key
      const int kr = min(kp0 + r, seq_len - 1) - kp0;
      const uint32_t unit = (uint32_t)(kr * a.H) * (D / 8) + (lseg ^ bswz<ROWB>(r));
      lds_dma16(kbase, unit, kd + j * 1024);
      lds_dma16(vbase, unit, vd + j * 1024);
    }
  };

  const uint32_t rbase = (uint32_t)(l32 * ROWB + ((hf ^ bswz<ROWB>(l32)) << 4));
  uint32_t tro[2][DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    tro[0][dt] = tr_offset<ROWB>(lane, dt, 0);
    tro[1][dt] = tr_offset<ROWB>(lane, dt, 1);
  }
  f32x16 dQT[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dQT[dt][r] = 0.f;

  // per-lane operand offsets held in registers; the chunk loop is unrolled
  // by buffer, so buffer and sub-chunk offsets ride in the LDS immediate
  auto opaque = [](uint32_t x) {
    asm volatile("" : "+v"(x));
    return x;
  };
  uint32_t aoff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) aoff[ks] = opaque(rbase ^ (ks << 5));
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    tro[0][dt] = opaque(tro[0][dt]);
    tro[1][dt] = opaque(tro[1][dt]);
  }
  auto chunk = [&](int ch, auto buf_t) {
    constexpr int BF = decltype(buf_t)::value;
    const int kp0 = key_lo + ch * kBwdChunk;
#pragma unroll
    for (int sc = 0; sc < 2; ++sc) {
      // the next chunk's loads go out after the first half's products, not
      // right after the barrier where every wave reads its first operands
      if (sc == 1 && ch + 1 < nchunks) load_chunk(ch + 1, BF ^ 1);
      const int ko = BF * BUF + sc * 32 * ROWB;  // compile-time after unrolling
      f32x16 S, dP;
#pragma unroll
      for (int r = 0; r < 16; ++r) { S[r] = 0.f; dP[r] = 0.f; }
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(smem + aoff[ks] + ko), qreg[ks], S, 0, 0, 0);
        dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            *reinterpret_cast<const bf16x8*>(smem + aoff[ks] + ko + CBYTES), oreg[ks], dP, 0, 0, 0);
      }
      // S[r], dP[r]: key kp0 + 32 sc + 8 (r / 4) + 4 hf + r % 4, query column l32
      const int kb = kp0 + 32 * sc + 4 * hf;
      const bool need_mask = MODE != kBwdHist && kp0 + 32 * sc + 31 > wq_min;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(fmaf(S[r], a.scale2, -lse2));
        if (need_mask && kb + 8 * (r >> 2) + (r & 3) > qpos) p = 0.f;
        dP[r] = p * (dP[r] - dq_d);
      }
      const bf16x8 s0 = regs_to_bf16(dP, 0), s1 = regs_to_bf16(dP, 1);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        dQT[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            tr_frag(smem + ko, tro[0][dt], tro[1][dt]), s0, dQT[dt], 0, 0, 0);
        dQT[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            tr_frag(smem + ko + 16 * ROWB, tro[0][dt], tro[1][dt]), s1, dQT[dt], 0, 0, 0);
      }
    }
    __syncthreads();  // chunk ch + 1 has landed; buffer BF is free again
  };
  using c0 = std::integral_constant<int, 0>;
  using c1 = std::integral_constant<int, 1>;
  load_chunk(0, 0);
  __syncthreads();
  int ch = 0;
  for (; ch + 2 <= nchunks; ch += 2) {
    chunk(ch, c0());
    chunk(ch + 1, c1());
  }
  if (ch < nchunks) chunk(ch, c0());

  // ---- dq += scale dQ: through LDS, so that each atomic instruction covers
  //      one query row's consecutive dims
  float* stg = (float*)smem + w * 32 * TS;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int m = 0; m < 4; ++m)
      *reinterpret_cast<f32x4*>(stg + l32 * TS + 32 * dt + 8 * m + 4 * hf) =
          f32x4{dQT[dt][4 * m] * a.scale, dQT[dt][4 * m + 1] * a.scale,
                dQT[dt][4 * m + 2] * a.scale, dQT[dt][4 * m + 3] * a.scale};
  // the wave's own region only: a wave-level LDS fence suffices
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (int r = 0; r < 32; ++r) {
    const int tok = __shfl(qtok, r);
    if (tok < 0) continue;  // uniform: the same row for the whole wave
    float* dst = a.dq + ((size_t)tok * a.H + h) * D;
    for (int e = lane; e < D; e += 64) unsafeAtomicAdd(dst + e, stg[r * TS + e]);
  }
}

// ---------------------------------------------------------------------------
// launches
// ---------------------------------------------------------------------------
hipError_t launch_bwd_prep(const void* out, bool out_f32, const uint16_t* dout, const float* lse,
                           const Geo& g, float* dvec, float* lse2, float* dq, hipStream_t st) {
  const long long rows = (long long)g.total_tokens * g.num_heads;
  if (rows == 0) return hipSuccess;
  dim3 grid((unsigned)((rows + 15) / 16));
#define MOBA_PREP(DD, F)                                                                     \
  hipLaunchKernelGGL((bwd_prep_kernel<DD, F>), grid, dim3(256), 0, st, out, dout, lse, rows, dvec, \
                     lse2, dq)
  if (g.head_dim == 128) {
    if (out_f32) MOBA_PREP(128, true); else MOBA_PREP(128, false);
  } else {
    if (out_f32) MOBA_PREP(64, true); else MOBA_PREP(64, false);
  }
#undef MOBA_PREP
  return hipGetLastError();
}

static BwdArgs bwd_args(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const uint16_t* dout, const float* lse, const float* dvec, const Geo& g,
                        int topk, float scale, const int32_t* list, const int32_t* offsets,
                        const int4* tile_info, float* dq, float* dk, float* dv) {
  BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.dvec = dvec;
  a.cu_seqlens = g.cu_seqlens;
  a.cu_blocks = g.cu_blocks;
  a.num_seqs = g.num_seqs;
  a.total_tokens = g.total_tokens;
  a.H = g.num_heads;
  a.block_size = g.block_size;
  a.topk = topk;
  a.NB = g.total_blocks;
  a.scale = scale;
  a.scale2 = scale * kLog2e;
  a.list = list;
  a.offsets = offsets;
  a.tile_info = tile_info;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.kgroups = g.block_size / kBwdKeysPerWg + (g.block_size % kBwdKeysPerWg ? 1 : 0);
  a.tiles_per_unit = (g.block_size + kBwdWaves * 32 - 1) / (kBwdWaves * 32);
  a.units_per_seq = (g.max_seqlen + g.block_size - 1) / g.block_size;
  return a;
}

hipError_t launch_bwd_kv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* dout, const float* lse, const float* dvec, const Geo& g,
                         int topk, float scale, const int32_t* list, const int32_t* offsets,
                         float* dk, float* dv, hipStream_t st) {
  if (g.total_blocks == 0) return hipSuccess;
  const BwdArgs a = bwd_args(q, k, v, dout, lse, dvec, g, topk, scale, list, offsets, nullptr,
                             nullptr, dk, dv);
  const long long n = (long long)g.num_heads * g.total_blocks * a.kgroups;
  dim3 grid((unsigned)n);
  if (g.head_dim == 128)
    hipLaunchKernelGGL(bwd_kv_pair_kernel<128>, grid, dim3(64 * kBwdPairWaves), 0, st, a);
  else
    hipLaunchKernelGGL(bwd_kv_pair_kernel<64>, grid, dim3(64 * kBwdPairWaves), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_bwd_q(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const uint16_t* dout, const float* lse, const float* dvec, const Geo& g,
                        int topk, float scale, const int32_t* list, const int4* tile_info,
                        long long hist_tiles, float* dq, hipStream_t st) {
  if (g.total_tokens == 0) return hipSuccess;
  const BwdArgs a = bwd_args(q, k, v, dout, lse, dvec, g, topk, scale, list, nullptr,
                             tile_info, dq, nullptr, nullptr);
  if (hist_tiles > 0) {
    dim3 grid((unsigned)hist_tiles);
    if (g.head_dim == 128)
      hipLaunchKernelGGL((bwd_q_kernel<128, kBwdHist>), grid, dim3(64 * kBwdWaves), 0, st, a);
    else
      hipLaunchKernelGGL((bwd_q_kernel<64, kBwdHist>), grid, dim3(64 * kBwdWaves), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid((unsigned)(g.num_seqs * a.units_per_seq * a.tiles_per_unit), g.num_heads);
  if (g.head_dim == 128)
    hipLaunchKernelGGL((bwd_q_kernel<128, kBwdOwn>), grid, dim3(64 * kBwdWaves), 0, st, a);
  else
    hipLaunchKernelGGL((bwd_q_kernel<64, kBwdOwn>), grid, dim3(64 * kBwdWaves), 0, st, a);
  return hipGetLastError();
}

}  // namespace moba
