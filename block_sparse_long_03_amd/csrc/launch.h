// Host-side launch wrappers shared between the kernel translation units and
// the C ABI layer.  All pointers are device pointers; nothing here allocates.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moba {

// num_heads is the head count of the [T, H, d] tensors (their row stride in
// heads).  A forward pass may run over one group of heads at a time:
// head_lo and head_cnt name the group, whose workspace arrays (partials,
// lists, staged V) are laid out for head_cnt heads and indexed by the head's
// place in the group.  Calls over all heads use head_lo 0, head_cnt num_heads.
struct Geo {
  const int32_t* cu_seqlens;
  const int32_t* cu_blocks;
  int num_seqs;
  int total_tokens;
  int max_seqlen;
  int total_blocks;
  int num_heads;
  int head_dim;
  int block_size;
  int head_lo;
  int head_cnt;
};

// Waves per workgroup of the MFMA attention kernels, one 32-query column
// tile per wave.  Long key ranges (block size >= 1024) use 8 waves: one
// 256-query tile per CU halves the K/V chunk traffic per flop.  Shorter ones
// use 4 waves: two 128-query workgroups per CU hide each other's tile
// start-up (list, query gather, first chunk).
constexpr int kMfmaWavesPerSimd = 2;
inline int mfma_waves(int key_range) { return key_range >= 1024 ? 8 : 4; }
inline int mfma_tile_q(int key_range) { return 32 * mfma_waves(key_range); }
constexpr int kF32TileQ = 1;

// Resident historical tiles: when a whole KV block fits in LDS (K and V^T of
// B keys: B * d * 4 bytes <= 128 KiB, e.g. B <= 256 at d = 128), an 8-wave
// workgroup loads it once and runs kResidentPasses passes of 256 gathered
// queries against it, so the block is fetched once per 4096 queries.
constexpr int kResidentLdsBytes = 128 * 1024;
constexpr int kResidentPasses = 16;
inline bool hist_resident(int block_size, int head_dim) {
  return (long long)block_size * head_dim * 4 <= kResidentLdsBytes;
}
// rows of one historical tile (one workgroup of the historical grid)
inline int hist_tile_q(int block_size, int head_dim) {
  return hist_resident(block_size, head_dim) ? 32 * 8 * kResidentPasses
                                             : mfma_tile_q(block_size);
}

// Workspace carve-up of moba_attn_fwd (offsets in bytes, 256-aligned).
struct AttnWorkspace {
  size_t counts, offsets, tile_offsets, list, lse_part, o_part, vt, tile_info, vmax, notfull,
      total;
};
AttnWorkspace attn_workspace_layout(bool bf16, long long total_tokens, long long total_blocks,
                                    long long num_heads, long long head_dim,
                                    long long block_size, long long topk);
// Upper bound on the number of historical tiles of hist_tile_q(block_size,
// head_dim) rows.
long long hist_tiles_bound(long long total_tokens, long long total_blocks, long long num_heads,
                           long long head_dim, long long block_size, long long topk);
size_t dense_workspace_bytes(bool bf16, long long total_blocks, long long num_heads,
                             long long head_dim, long long block_size);

// kbar3 (optional): the means as hi + mid + lo bf16 planes [block, head, 3, d]
hipError_t launch_pool_keys(const void* k, bool bf16, const Geo& g, float* kbar,
                            uint16_t* kbar3, hipStream_t st);
// bf16 queries score against kbar3, fp32 queries against kbar
hipError_t launch_gate_topk(const void* q, bool bf16, const float* kbar, const uint16_t* kbar3,
                            const Geo& g, int topk, int32_t* block_idx, hipStream_t st);
hipError_t launch_pool_minmax(const void* k, bool bf16, const Geo& g, float* kmm, hipStream_t st);
hipError_t launch_gate_topk_minmax(const uint16_t* q, const float* kmm, const Geo& g, int topk,
                                   int32_t* block_idx, hipStream_t st);
hipError_t launch_static_select(const Geo& g, int topk, int sink, int32_t* block_idx,
                                hipStream_t st);

// Query bucketing: counts per (head, KV block), exclusive scans of entries and
// of tiles, and the scatter of (token, slot) entries into per-block lists.
// With tile_info, also writes {key, first entry, end entry, 0} for each of
// the max_tiles tiles of tile_q rows (key -1 past the last tile).
// List entries are token * topk + slot, or (tokens_only) the global token.
// dense_blocks > 0: rows of the dense prefix (dense_row in common.h) get no
// entries, and notfull[head of the group, global block] is set to 1 for
// every block below dense_blocks holding a row that is not one.
hipError_t launch_bucket(const int32_t* block_idx, const Geo& g, int topk, int tile_q,
                         int32_t* counts, int32_t* offsets, int32_t* tile_offsets,
                         int32_t* list, int4* tile_info, long long max_tiles, hipStream_t st,
                         bool tokens_only = false, int dense_blocks = 0,
                         int32_t* notfull = nullptr);

// Transposed, key-permuted fp16 copy of V per (block, head) for the MFMA
// kernels, scaled per head by 2^-e (vmax_bits[h] receives max |v|).
hipError_t launch_v_transpose(const void* v, const Geo& g, uint32_t* vmax_bits, uint16_t* vt,
                              hipStream_t st);

// bf16 MFMA attention.  mode: 0 historical blocks (gathered queries, partials),
// 1 own block (causal, partials), 2 dense causal (final output).
// Partials (hist, own) are fp16 in the staged V's units; dense scales back.
hipError_t launch_attn_mfma_hist(const void* q, const void* k, const uint16_t* vt,
                                 const Geo& g, int topk, float scale, const int32_t* list,
                                 const int4* tile_info, long long max_tiles, uint16_t* o_part,
                                 float* lse_part, hipStream_t st);
// own: blocks below dense_blocks whose notfull flag is 0 hold only
// dense-prefix rows and are skipped.  dense: queries at local positions
// below q_limit only (the dense prefix of each sequence; INT_MAX: all).
hipError_t launch_attn_mfma_own(const void* q, const void* k, const uint16_t* vt,
                                const Geo& g, int topk, float scale, uint16_t* o_part,
                                float* lse_part, int dense_blocks, const int32_t* notfull,
                                hipStream_t st);
// Workgroups of a dense launch over the first q_limit positions of each
// sequence (every sequence padded to the longest one) and all num_heads
// heads.  It depends on the layer's geometry only, not on how the heads are
// split into passes, so a choice made from it is the same for every split.
inline long long dense_grid(const Geo& g, int q_limit) {
  const int span = q_limit < g.max_seqlen ? q_limit : g.max_seqlen;
  if (span <= 0) return 0;
  const int tq = mfma_tile_q(span);
  return (long long)((span + tq - 1) / tq) * g.num_seqs * g.num_heads;
}
hipError_t launch_attn_mfma_dense(const void* q, const void* k, const uint16_t* vt,
                                  const uint32_t* vmax_bits, const Geo& g, float scale,
                                  void* out, bool out_bf16, float* lse, hipStream_t st,
                                  int q_limit = 0x7fffffff);

// fp32 VALU attention (one wave per query row and key range).
hipError_t launch_attn_f32_hist(const float* q, const float* k, const float* v, const Geo& g,
                                int topk, float scale, const int32_t* list,
                                const int32_t* offsets, long long max_entries, float* o_part,
                                float* lse_part, hipStream_t st);
hipError_t launch_attn_f32_own(const float* q, const float* k, const float* v, const Geo& g,
                               int topk, float scale, float* o_part, float* lse_part,
                               hipStream_t st);
hipError_t launch_attn_f32_dense(const float* q, const float* k, const float* v, const Geo& g,
                                 float scale, void* out, bool out_bf16, float* lse,
                                 hipStream_t st);

// Online-softmax combine of the partials of every (token, head) row (rows of
// the dense prefix excepted when dense_blocks > 0).
hipError_t launch_merge(const int32_t* block_idx, const Geo& g, int topk, int dense_blocks,
                        const void* o_part, bool part_f16, const float* lse_part,
                        const uint32_t* vmax_bits, void* out, bool out_bf16, float* lse,
                        hipStream_t st);

// Backward: Dq = rowsum(dO * O) and dq = 0; dK, dV per (head, block, 128
// keys) over the block's list and own-block queries; dQ over the forward's
// historical tiles (tile_info) and own-block tiles, added to dq atomically.
// dvec = rowsum(dout * out), lse2 = lse log2(e) (read by bwd_kv), dq = 0
hipError_t launch_bwd_prep(const void* out, bool out_f32, const uint16_t* dout, const float* lse,
                           const Geo& g, float* dvec, float* lse2, float* dq, hipStream_t st);
// lse2: lse log2(e), as bwd_prep writes it
hipError_t launch_bwd_kv(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const uint16_t* dout, const float* lse2, const float* dvec, const Geo& g,
                         int topk, float scale, const int32_t* list, const int32_t* offsets,
                         float* dk, float* dv, hipStream_t st);
hipError_t launch_bwd_q(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                        const uint16_t* dout, const float* lse, const float* dvec, const Geo& g,
                        int topk, float scale, const int32_t* list, const int4* tile_info,
                        long long hist_tiles, float* dq, hipStream_t st);

// The device address of the library's fixed workspace on the current device
// (MOBA_STATIC_WORKSPACE_BYTES, looked up once per device) and its size.
hipError_t static_workspace(void** ptr, size_t* bytes);

// Measurement support: `workgroups` x 4 waves, each running 4 independent
// chains of `iterations` 32x32x16 bf16 MFMAs (2 * 32 * 32 * 16 flops each);
// operands 0 = fixed register operands, 1 = random register operands,
// 2 = random operands with B read from LDS (iterations a multiple of 8 for
// 1 and 2); sink holds workgroups * 256 floats.
hipError_t launch_mfma_rate(int workgroups, int iterations, int operands, float* sink,
                            hipStream_t st);

}  // namespace moba
