// C ABI of libmoba.so: host-side validation, workspace carve-up and launch
// order.  See include/moba.h for the contract of every entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/moba.h"
#include "launch.h"

struct moba_profiler {
  struct Rec {
    std::string name;
    hipEvent_t start, stop;
  };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> spare;
};

namespace {

thread_local int g_last_hip_error = 0;
thread_local moba_profiler* g_profiler = nullptr;

hipEvent_t profiler_event(moba_profiler* p) {
  if (!p->spare.empty()) {
    hipEvent_t e = p->spare.back();
    p->spare.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs one launch group; with a profiler attached, brackets it with events.
template <class F>
hipError_t timed(const char* name, hipStream_t s, F&& launch) {
  moba_profiler* p = g_profiler;
  if (!p) return launch();
  hipEvent_t a = profiler_event(p), b = profiler_event(p);
  if (!a || !b) return launch();
  (void)hipEventRecord(a, s);
  hipError_t e = launch();
  (void)hipEventRecord(b, s);
  p->recs.push_back({name, a, b});
  return e;
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

moba_status hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return MOBA_ERR_HIP;
}

bool dtype_ok(int dt) { return dt == MOBA_F32 || dt == MOBA_BF16; }

// Checks of the shared geometry arguments.  Nothing here touches the device.
moba_status check_geometry(int dtype, const int32_t* cu_seqlens, const int32_t* cu_blocks,
                           int num_seqs, int total_tokens, int max_seqlen, int total_blocks,
                           int num_heads, int head_dim, int block_size) {
  if (!cu_seqlens || !cu_blocks) return MOBA_ERR_INVALID_ARG;
  if (!dtype_ok(dtype)) return MOBA_ERR_INVALID_ARG;
  if (num_seqs < 1 || total_tokens < 0 || max_seqlen < 0 || total_blocks < 0)
    return MOBA_ERR_INVALID_ARG;
  if (num_heads < 1 || head_dim < 1 || block_size < 1) return MOBA_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return MOBA_ERR_UNSUPPORTED;
  if (block_size % 64 != 0) return MOBA_ERR_UNSUPPORTED;
  if (max_seqlen > total_tokens) return MOBA_ERR_INVALID_ARG;
  if (total_tokens > 0) {
    if (max_seqlen < 1) return MOBA_ERR_INVALID_ARG;
    if ((long long)max_seqlen * num_seqs < total_tokens) return MOBA_ERR_INVALID_ARG;
    const long long min_blocks = ((long long)total_tokens + block_size - 1) / block_size;
    if (total_blocks < min_blocks || total_blocks > total_tokens) return MOBA_ERR_INVALID_ARG;
    if (total_blocks < (max_seqlen + block_size - 1) / block_size) return MOBA_ERR_INVALID_ARG;
  } else if (total_blocks != 0) {
    return MOBA_ERR_INVALID_ARG;
  }
  // 32-bit limits of the launch grids and of the packed list entries
  if ((long long)num_heads * total_blocks + 1 >= (1LL << 31)) return MOBA_ERR_UNSUPPORTED;
  if ((long long)total_blocks * (block_size / 64) >= (1LL << 31)) return MOBA_ERR_UNSUPPORTED;
  if ((long long)num_seqs * ((max_seqlen + 63) / 64) >= (1LL << 31)) return MOBA_ERR_UNSUPPORTED;
  if ((long long)total_tokens * num_heads >= (1LL << 33)) return MOBA_ERR_UNSUPPORTED;
  if (num_heads > 65535) return MOBA_ERR_UNSUPPORTED;
  return MOBA_OK;
}

moba_status check_topk(int total_tokens, int topk) {
  if (topk < 1) return MOBA_ERR_INVALID_ARG;
  if (topk > 64) return MOBA_ERR_UNSUPPORTED;
  if ((long long)total_tokens * topk >= (1LL << 31)) return MOBA_ERR_UNSUPPORTED;
  return MOBA_OK;
}

moba::Geo make_geo(const int32_t* cu_seqlens, const int32_t* cu_blocks, int num_seqs,
                   int total_tokens, int max_seqlen, int total_blocks, int num_heads,
                   int head_dim, int block_size) {
  moba::Geo g;
  g.cu_seqlens = cu_seqlens;
  g.cu_blocks = cu_blocks;
  g.num_seqs = num_seqs;
  g.total_tokens = total_tokens;
  g.max_seqlen = max_seqlen;
  g.total_blocks = total_blocks;
  g.num_heads = num_heads;
  g.head_dim = head_dim;
  g.block_size = block_size;
  g.head_lo = 0;
  g.head_cnt = num_heads;
  return g;
}

// historical list entries and tiles of one pass over the heads of g's group
long long hist_entries_bound(const moba::Geo& g, int topk) {
  return (long long)g.total_tokens * g.head_cnt * (topk - 1);
}

long long hist_tiles_bound(const moba::Geo& g, int topk) {
  return moba::hist_tiles_bound(g.total_tokens, g.total_blocks, g.head_cnt, g.head_dim,
                                g.block_size, topk);
}

// heads per pass of moba_attn_fwd: 0 or anything above num_heads means all
int heads_per_pass(int num_heads, int head_chunk) {
  return (head_chunk <= 0 || head_chunk > num_heads) ? num_heads : head_chunk;
}

// 32-bit limits of one pass: list entries (and their offsets), the tile
// grid, and the packed entries token * topk + slot
bool pass_fits_int32(const moba::Geo& g, int topk) {
  return hist_tiles_bound(g, topk) < (1LL << 31) && hist_entries_bound(g, topk) < (1LL << 31);
}

}  // namespace

namespace moba {

long long hist_tiles_bound(long long T, long long NB, long long H, long long D, long long B,
                           long long topk) {
  if (topk < 2) return 0;
  const long long e = T * H * (topk - 1);
  const long long tq = hist_tile_q((int)B, (int)D);
  return (e + tq - 1) / tq + H * NB;
}

// Backward workspace: the bucket lists and tiles of 128 queries, and
// Dq = rowsum(dO * O) per (token, head).
struct BwdWorkspace {
  size_t counts, offsets, tile_offsets, list, tile_info, dvec, lse2, total;
};

constexpr int kBwdTileQ = 128;
// one workgroup per CU
constexpr long long kPrefixMinGrid = 256;

long long bwd_tiles_bound(long long T, long long NB, long long H, long long topk) {
  if (topk < 2) return 0;
  return (T * H * (topk - 1) + kBwdTileQ - 1) / kBwdTileQ + H * NB;
}

BwdWorkspace bwd_workspace_layout(long long T, long long NB, long long H, long long topk) {
  BwdWorkspace w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  const size_t nkeys = (size_t)(H * NB);
  w.counts = take(nkeys * 4);
  w.offsets = take((nkeys + 1) * 4);
  w.tile_offsets = take((nkeys + 1) * 4);
  w.list = take((size_t)(T * H * (topk > 1 ? topk - 1 : 1)) * 4);
  w.tile_info = take((size_t)bwd_tiles_bound(T, NB, H, topk) * 16);
  w.dvec = take((size_t)(T * H) * 4);
  w.lse2 = take((size_t)(T * H) * 4);
  w.total = off;
  return w;
}

AttnWorkspace attn_workspace_layout(bool bf16, long long T, long long NB, long long H,
                                    long long D, long long B, long long topk) {
  AttnWorkspace w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  const size_t nkeys = (size_t)(H * NB);
  w.counts = take(nkeys * 4);
  w.offsets = take((nkeys + 1) * 4);
  w.tile_offsets = take((nkeys + 1) * 4);
  w.list = take((size_t)(T * H * (topk > 1 ? topk - 1 : 1)) * 4);
  w.lse_part = take((size_t)(T * H * topk) * 4);
  w.o_part = take((size_t)(T * H * topk * D) * (bf16 ? 2 : 4));
  w.vt = take(bf16 ? (size_t)(NB * B * H * D) * 2 : 0);
  w.tile_info = take(bf16 ? (size_t)hist_tiles_bound(T, NB, H, D, B, topk) * 16 : 0);
  w.vmax = take((size_t)H * 4);
  w.notfull = take(bf16 ? nkeys * 4 : 0);
  w.total = off;
  return w;
}

size_t dense_workspace_bytes(bool bf16, long long NB, long long H, long long D, long long B) {
  if (!bf16) return kAlign;  // the fp32 path stages nothing
  return align_up((size_t)(NB * B * H * D) * 2) + align_up((size_t)H * 4) + kAlign;
}

}  // namespace moba

namespace {

// One pass of moba_attn_fwd over the heads of g's group: V staging, bucketing,
// historical and own-block attention into the group's partials, merge into
// out and lse.  bf16: rows of a sequence's first topk blocks that select every
// earlier block (all of them under the gate) attend to their whole causal
// prefix, so the dense kernel writes them directly (stage "attn_prefix") and
// bucketing, the own-block pass and the merge skip them.  This route is taken
// when the prefix launch over all heads fills the chip (kPrefixMinGrid
// workgroups): a smaller one runs for as long as its heaviest tile (topk *
// block_size keys) takes, longer than the passes it saves.  The choice does
// not depend on the head passes, so neither do the results.
moba_status attn_pass(const void* q, const void* k, const void* v, bool bf16, const moba::Geo& g,
                      int topk, const int32_t* block_idx, float softmax_scale, void* out,
                      int out_dtype, float* lse, char* ws, const moba::AttnWorkspace& L,
                      hipStream_t s) {
  const long long tiles = hist_tiles_bound(g, topk);
  int32_t* counts = (int32_t*)(ws + L.counts);
  int32_t* offsets = (int32_t*)(ws + L.offsets);
  int32_t* tile_offsets = (int32_t*)(ws + L.tile_offsets);
  int32_t* list = (int32_t*)(ws + L.list);
  float* lse_part = (float*)(ws + L.lse_part);
  void* o_part = ws + L.o_part;
  uint32_t* vmax = (uint32_t*)(ws + L.vmax);
  const bool out_bf16 = out_dtype == MOBA_BF16;
  hipError_t e;
  int dense_blocks = 0;  // rows of blocks below it may take the dense-prefix route

  if (bf16) {
    uint16_t* vt = (uint16_t*)(ws + L.vt);
    int4* tile_info = (int4*)(ws + L.tile_info);
    int32_t* notfull = (int32_t*)(ws + L.notfull);
    const int q_limit = (int)std::min<long long>((long long)topk * g.block_size, INT_MAX);
    if (moba::dense_grid(g, q_limit) >= moba::kPrefixMinGrid) dense_blocks = topk;
    if ((e = timed("v_stage", s, [&] { return moba::launch_v_transpose(v, g, vmax, vt, s); })) !=
        hipSuccess)
      return hip_fail(e);
    if ((e = timed("bucket", s, [&] {
           return moba::launch_bucket(block_idx, g, topk,
                                      moba::hist_tile_q(g.block_size, g.head_dim), counts,
                                      offsets, tile_offsets, list, tile_info, tiles, s, false,
                                      dense_blocks, notfull);
         })) != hipSuccess)
      return hip_fail(e);
    if (dense_blocks > 0 &&
        (e = timed("attn_prefix", s, [&] {
           return moba::launch_attn_mfma_dense(q, k, vt, vmax, g, softmax_scale, out, out_bf16,
                                               lse, s, q_limit);
         })) != hipSuccess)
      return hip_fail(e);
    if ((e = timed("attn_hist", s, [&] {
           return moba::launch_attn_mfma_hist(q, k, vt, g, topk, softmax_scale, list,
                                              tile_info, tiles, (uint16_t*)o_part, lse_part, s);
         })) != hipSuccess)
      return hip_fail(e);
    if ((e = timed("attn_own", s, [&] {
           return moba::launch_attn_mfma_own(q, k, vt, g, topk, softmax_scale,
                                             (uint16_t*)o_part, lse_part, dense_blocks,
                                             notfull, s);
         })) != hipSuccess)
      return hip_fail(e);
  } else {
    if ((e = timed("bucket", s, [&] {
           return moba::launch_bucket(block_idx, g, topk, moba::kF32TileQ, counts, offsets,
                                      tile_offsets, list, nullptr, 0, s);
         })) != hipSuccess)
      return hip_fail(e);
    if ((e = timed("attn_hist", s, [&] {
           return moba::launch_attn_f32_hist((const float*)q, (const float*)k, (const float*)v,
                                             g, topk, softmax_scale, list, offsets,
                                             hist_entries_bound(g, topk), (float*)o_part,
                                             lse_part, s);
         })) != hipSuccess)
      return hip_fail(e);
    if ((e = timed("attn_own", s, [&] {
           return moba::launch_attn_f32_own((const float*)q, (const float*)k, (const float*)v,
                                            g, topk, softmax_scale, (float*)o_part, lse_part, s);
         })) != hipSuccess)
      return hip_fail(e);
  }
  if ((e = timed("merge", s, [&] {
         return moba::launch_merge(block_idx, g, topk, dense_blocks, o_part, bf16, lse_part,
                                   vmax, out, out_bf16, lse, s);
       })) != hipSuccess)
    return hip_fail(e);
  return MOBA_OK;
}

}  // namespace

extern "C" {

int moba_api_version(void) { return MOBA_API_VERSION; }

const char* moba_status_str(int status) {
  switch (status) {
    case MOBA_OK: return "MOBA_OK";
    case MOBA_ERR_INVALID_ARG: return "MOBA_ERR_INVALID_ARG";
    case MOBA_ERR_UNSUPPORTED: return "MOBA_ERR_UNSUPPORTED";
    case MOBA_ERR_WORKSPACE_TOO_SMALL: return "MOBA_ERR_WORKSPACE_TOO_SMALL";
    case MOBA_ERR_HIP: return "MOBA_ERR_HIP";
    default: return "MOBA_ERR_UNKNOWN";
  }
}

int moba_last_hip_error(void) { return g_last_hip_error; }

moba_status moba_pool_keys(const void* k, int dtype, const int32_t* cu_seqlens,
                           const int32_t* cu_blocks, int num_seqs, int total_tokens,
                           int max_seqlen, int total_blocks, int num_heads, int head_dim,
                           int block_size, float* kbar, uint16_t* kbar3, void* stream) {
  moba_status st = check_geometry(dtype, cu_seqlens, cu_blocks, num_seqs, total_tokens,
                                  max_seqlen, total_blocks, num_heads, head_dim, block_size);
  if (st != MOBA_OK) return st;
  if (total_tokens == 0) return MOBA_OK;
  if (!k || !kbar) return MOBA_ERR_INVALID_ARG;
  moba::Geo g = make_geo(cu_seqlens, cu_blocks, num_seqs, total_tokens, max_seqlen,
                         total_blocks, num_heads, head_dim, block_size);
  hipError_t e = timed("pool_keys", (hipStream_t)stream, [&] {
    return moba::launch_pool_keys(k, dtype == MOBA_BF16, g, kbar, kbar3, (hipStream_t)stream);
  });
  return e == hipSuccess ? MOBA_OK : hip_fail(e);
}

moba_status moba_gate_topk(const void* q, int dtype, const float* kbar,
                           const uint16_t* kbar3, const int32_t* cu_seqlens,
                           const int32_t* cu_blocks, int num_seqs,
                           int total_tokens, int max_seqlen, int total_blocks, int num_heads,
                           int head_dim, int block_size, int topk, int32_t* block_idx,
                           void* stream) {
  moba_status st = check_geometry(dtype, cu_seqlens, cu_blocks, num_seqs, total_tokens,
                                  max_seqlen, total_blocks, num_heads, head_dim, block_size);
  if (st != MOBA_OK) return st;
  st = check_topk(total_tokens, topk);
  if (st != MOBA_OK) return st;
  if (total_tokens == 0) return MOBA_OK;
  const bool bf16 = dtype == MOBA_BF16;
  if (!q || !block_idx || (bf16 ? !kbar3 : !kbar)) return MOBA_ERR_INVALID_ARG;
  moba::Geo g = make_geo(cu_seqlens, cu_blocks, num_seqs, total_tokens, max_seqlen,
                         total_blocks, num_heads, head_dim, block_size);
  hipError_t e = timed("gate_topk", (hipStream_t)stream, [&] {
    return moba::launch_gate_topk(q, bf16, kbar, kbar3, g, topk, block_idx,
                                  (hipStream_t)stream);
  });
  return e == hipSuccess ? MOBA_OK : hip_fail(e);
}

moba_status moba_pool_minmax(const void* k, int dtype, const int32_t* cu_seqlens,
                             const int32_t* cu_blocks, int num_seqs, int total_tokens,
                             int max_seqlen, int total_blocks, int num_heads, int head_dim,
                             int block_size, float* kminmax, void* stream) {
  moba_status st = check_geometry(dtype, cu_seqlens, cu_blocks, num_seqs, total_tokens,
                                  max_seqlen, total_blocks, num_heads, head_dim, block_size);
  if (st != MOBA_OK) return st;
  if (total_tokens == 0) return MOBA_OK;
  if (!k || !kminmax) return MOBA_ERR_INVALID_ARG;
  moba::Geo g = make_geo(cu_seqlens, cu_blocks, num_seqs, total_tokens, max_seqlen,
                         total_blocks, num_heads, head_dim, block_size);
  hipError_t e = timed("pool_minmax", (hipStream_t)stream, [&] {
    return moba::launch_pool_minmax(k, dtype == MOBA_BF16, g, kminmax, (hipStream_t)stream);
  });
  return e == hipSuccess ? MOBA_OK : hip_fail(e);
}

moba_status moba_gate_topk_minmax(const void* q, int dtype, const float* kminmax,
                                  const int32_t* cu_seqlens, const int32_t* cu_blocks,
                                  int num_seqs, int total_tokens, int max_seqlen,
                                  int total_blocks, int num_heads, int head_dim, int block_size,
                                  int topk, int32_t* block_idx, void* stream) {
  moba_status st = check_geometry(dtype, cu_seqlens, cu_blocks, num_seqs, total_tokens,
                                  max_seqlen, total_blocks, num_heads, head_dim, block_size);
  if (st != MOBA_OK) return st;
  st = check_topk(total_tokens, topk);
  if (st != MOBA_OK) return st;
  if (dtype != MOBA_BF16) return MOBA_ERR_UNSUPPORTED;
  if (total_tokens == 0) return MOBA_OK;
  if (!q || !kminmax || !block_idx) return MOBA_ERR_INVALID_ARG;
  moba::Geo g = make_geo(cu_seqlens, cu_blocks, num_seqs, total_tokens, max_seqlen,
                         total_blocks, num_heads, head_dim, block_size);
  hipError_t e = timed("gate_topk_minmax", (hipStream_t)stream, [&] {
    return moba::launch_gate_topk_minmax((const uint16_t*)q, kminmax, g, topk, block_idx,
                                         (hipStream_t)stream);
  });
  return e == hipSuccess ? MOBA_OK : hip_fail(e);
}

moba_status moba_static_select(const int32_t* cu_seqlens, const int32_t* cu_blocks,
                               int num_seqs, int total_tokens, int max_seqlen, int total_blocks,
                               int num_heads, int block_size, int topk, int sink_blocks,
                               int32_t* block_idx, void* stream) {
  // the selection does not depend on dtype or head_dim: any supported pair
  // checks the rest of the geometry
  moba_status st = check_geometry(MOBA_BF16, cu_seqlens, cu_blocks, num_seqs, total_tokens,
                                  max_seqlen, total_blocks, num_heads, 64, block_size);
  if (st != MOBA_OK) return st;
  st = check_topk(total_tokens, topk);
  if (st != MOBA_OK) return st;
  if (sink_blocks < 0) return MOBA_ERR_INVALID_ARG;
  if (total_tokens == 0) return MOBA_OK;
  if (!block_idx) return MOBA_ERR_INVALID_ARG;
  moba::Geo g = make_geo(cu_seqlens, cu_blocks, num_seqs, total_tokens, max_seqlen,
                         total_blocks, num_heads, 64, block_size);
  hipError_t e = timed("static_select", (hipStream_t)stream, [&] {
    return moba::launch_static_select(g, topk, sink_blocks, block_idx, (hipStream_t)stream);
  });
  return e == hipSuccess ? MOBA_OK : hip_fail(e);
}

size_t moba_attn_workspace_bytes(int dtype, int total_tokens, int total_blocks, int num_heads,
                                 int head_dim, int block_size, int topk, int head_chunk) {
  if (!dtype_ok(dtype) || total_tokens < 0 || total_blocks < 0 || num_heads < 1 ||
      (head_dim != 64 && head_dim != 128) || block_size < 64 || block_size % 64 != 0 ||
      head_chunk < 0 || check_topk(total_tokens, topk) != MOBA_OK)
    return 0;
  return moba::attn_workspace_layout(dtype == MOBA_BF16, total_tokens, total_blocks,
                                     heads_per_pass(num_heads, head_chunk), head_dim,
                                     block_size, topk)
      .total + kAlign;
}

moba_status moba_attn_fwd(const void* q, const void* k, const void* v, int dtype,
                          const int32_t* cu_seqlens, const int32_t* cu_blocks, int num_seqs,
                          int total_tokens, int max_seqlen, int total_blocks, int num_heads,
                          int head_dim, int block_size, int topk, const int32_t* block_idx,
                          float softmax_scale, void* out, int out_dtype, float* lse,
                          int head_chunk, void* workspace, size_t workspace_bytes,
                          void* stream) {
  moba_status st = check_geometry(dtype, cu_seqlens, cu_blocks, num_seqs, total_tokens,
                                  max_seqlen, total_blocks, num_heads, head_dim, block_size);
  if (st != MOBA_OK) return st;
  st = check_topk(total_tokens, topk);
  if (st != MOBA_OK) return st;
  if (!dtype_ok(out_dtype)) return MOBA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return MOBA_ERR_INVALID_ARG;
  if (head_chunk < 0) return MOBA_ERR_INVALID_ARG;
  const int hc = heads_per_pass(num_heads, head_chunk);
  moba::Geo g = make_geo(cu_seqlens, cu_blocks, num_seqs, total_tokens, max_seqlen,
                         total_blocks, num_heads, head_dim, block_size);
  g.head_cnt = hc;
  if (!pass_fits_int32(g, topk)) return MOBA_ERR_UNSUPPORTED;
  if (total_tokens == 0) return MOBA_OK;
  if (!q || !k || !v || !block_idx || !out || !lse || !workspace) return MOBA_ERR_INVALID_ARG;
  if ((uintptr_t)workspace % kAlign != 0) return MOBA_ERR_INVALID_ARG;
  const bool bf16 = dtype == MOBA_BF16;
  const moba::AttnWorkspace L = moba::attn_workspace_layout(
      bf16, total_tokens, total_blocks, hc, head_dim, block_size, topk);
  if (workspace_bytes < L.total) return MOBA_ERR_WORKSPACE_TOO_SMALL;
  for (int h0 = 0; h0 < num_heads; h0 += hc) {
    g.head_lo = h0;
    g.head_cnt = std::min(hc, num_heads - h0);
    st = attn_pass(q, k, v, bf16, g, topk, block_idx, softmax_scale, out, out_dtype, lse,
                   (char*)workspace, L, (hipStream_t)stream);
    if (st != MOBA_OK) return st;
  }
  return MOBA_OK;
}

moba_status moba_attn_fwd_static(const void* q, const void* k, const void* v, int dtype,
                                 const int32_t* cu_seqlens, const int32_t* cu_blocks,
                                 int num_seqs, int total_tokens, int max_seqlen,
                                 int total_blocks, int num_heads, int head_dim,
                                 int block_size, int topk, const int32_t* block_idx,
                                 float softmax_scale, void* out, int out_dtype, float* lse,
                                 void* stream) {
  // everything that can be checked without the device first: an invalid or
  // oversized call touches nothing
  moba_status st = check_geometry(dtype, cu_seqlens, cu_blocks, num_seqs, total_tokens,
                                  max_seqlen, total_blocks, num_heads, head_dim, block_size);
  if (st != MOBA_OK) return st;
  st = check_topk(total_tokens, topk);
  if (st != MOBA_OK) return st;
  if (!dtype_ok(out_dtype)) return MOBA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return MOBA_ERR_INVALID_ARG;
  if (total_tokens == 0) return MOBA_OK;
  if (!q || !k || !v || !block_idx || !out || !lse) return MOBA_ERR_INVALID_ARG;
  // the most heads per pass whose workspace fits the fixed array
  const bool bf16 = dtype == MOBA_BF16;
  auto need = [&](int hc) {
    return moba::attn_workspace_layout(bf16, total_tokens, total_blocks, hc, head_dim,
                                       block_size, topk)
        .total;
  };
  const size_t one = need(1);
  if (one > (size_t)MOBA_STATIC_WORKSPACE_BYTES) return MOBA_ERR_WORKSPACE_TOO_SMALL;
  int hc = (int)std::min<size_t>((size_t)num_heads, (size_t)MOBA_STATIC_WORKSPACE_BYTES / one);
  while (hc > 1 && need(hc) > (size_t)MOBA_STATIC_WORKSPACE_BYTES) --hc;
  void* ws = nullptr;
  size_t ws_bytes = 0;
  hipError_t e = moba::static_workspace(&ws, &ws_bytes);
  if (e != hipSuccess) return hip_fail(e);
  return moba_attn_fwd(q, k, v, dtype, cu_seqlens, cu_blocks, num_seqs, total_tokens,
                       max_seqlen, total_blocks, num_heads, head_dim, block_size, topk,
                       block_idx, softmax_scale, out, out_dtype, lse, hc, ws, ws_bytes, stream);
}

size_t moba_attn_bwd_workspace_bytes(int dtype, int total_tokens, int total_blocks,
                                     int num_heads, int head_dim, int block_size, int topk) {
  if (dtype != MOBA_BF16 || total_tokens < 0 || total_blocks < 0 || num_heads < 1 ||
      (head_dim != 64 && head_dim != 128) || block_size < 64 || block_size % 64 != 0 ||
      check_topk(total_tokens, topk) != MOBA_OK)
    return 0;
  return moba::bwd_workspace_layout(total_tokens, total_blocks, num_heads, topk).total + kAlign;
}

moba_status moba_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                          int out_dtype, const void* dout, const float* lse, int dtype,
                          const int32_t* cu_seqlens, const int32_t* cu_blocks, int num_seqs,
                          int total_tokens, int max_seqlen, int total_blocks, int num_heads,
                          int head_dim, int block_size, int topk, const int32_t* block_idx,
                          float softmax_scale, float* dq, float* dk, float* dv, void* workspace,
                          size_t workspace_bytes, void* stream) {
  moba_status st = check_geometry(dtype, cu_seqlens, cu_blocks, num_seqs, total_tokens,
                                  max_seqlen, total_blocks, num_heads, head_dim, block_size);
  if (st != MOBA_OK) return st;
  st = check_topk(total_tokens, topk);
  if (st != MOBA_OK) return st;
  if (dtype != MOBA_BF16) return MOBA_ERR_UNSUPPORTED;
  if (!dtype_ok(out_dtype)) return MOBA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return MOBA_ERR_INVALID_ARG;
  if (total_tokens == 0) return MOBA_OK;
  if (!q || !k || !v || !out || !dout || !lse || !block_idx || !dq || !dk || !dv || !workspace)
    return MOBA_ERR_INVALID_ARG;
  if ((uintptr_t)workspace % kAlign != 0) return MOBA_ERR_INVALID_ARG;
  const moba::BwdWorkspace L =
      moba::bwd_workspace_layout(total_tokens, total_blocks, num_heads, topk);
  if (workspace_bytes < L.total) return MOBA_ERR_WORKSPACE_TOO_SMALL;
  const long long tiles = moba::bwd_tiles_bound(total_tokens, total_blocks, num_heads, topk);
  moba::Geo g = make_geo(cu_seqlens, cu_blocks, num_seqs, total_tokens, max_seqlen,
                         total_blocks, num_heads, head_dim, block_size);
  if (tiles >= (1LL << 31) || hist_entries_bound(g, topk) >= (1LL << 31))
    return MOBA_ERR_UNSUPPORTED;
  char* ws = (char*)workspace;
  int32_t* counts = (int32_t*)(ws + L.counts);
  int32_t* offsets = (int32_t*)(ws + L.offsets);
  int32_t* tile_offsets = (int32_t*)(ws + L.tile_offsets);
  int32_t* list = (int32_t*)(ws + L.list);
  int4* tile_info = (int4*)(ws + L.tile_info);
  float* dvec = (float*)(ws + L.dvec);
  float* lse2 = (float*)(ws + L.lse2);
  const uint16_t *qb = (const uint16_t*)q, *kb = (const uint16_t*)k, *vb = (const uint16_t*)v,
                 *gb = (const uint16_t*)dout;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if ((e = timed("bwd_prep", s, [&] {
         return moba::launch_bwd_prep(out, out_dtype == MOBA_F32, gb, lse, g, dvec, lse2, dq, s);
       })) != hipSuccess)
    return hip_fail(e);
  if ((e = timed("bucket", s, [&] {
         return moba::launch_bucket(block_idx, g, topk, moba::kBwdTileQ, counts, offsets,
                                    tile_offsets, list, tile_info, tiles, s,
                                    /*tokens_only=*/true);
       })) != hipSuccess)
    return hip_fail(e);
  if ((e = timed("bwd_kv", s, [&] {
         return moba::launch_bwd_kv(qb, kb, vb, gb, lse2, dvec, g, topk, softmax_scale, list,
                                    offsets, dk, dv, s);
       })) != hipSuccess)
    return hip_fail(e);
  if ((e = timed("bwd_q", s, [&] {
         return moba::launch_bwd_q(qb, kb, vb, gb, lse, dvec, g, topk, softmax_scale, list,
                                   tile_info, tiles, dq, s);
       })) != hipSuccess)
    return hip_fail(e);
  return MOBA_OK;
}

moba_status moba_probe_mfma_rate(int workgroups, int iterations, int operands, float* sink,
                                 void* stream) {
  if (workgroups < 1 || iterations < 1 || !sink || operands < 0 || operands > 2 ||
      (operands != 0 && iterations % 8 != 0))
    return MOBA_ERR_INVALID_ARG;
  hipError_t e =
      moba::launch_mfma_rate(workgroups, iterations, operands, sink, (hipStream_t)stream);
  return e == hipSuccess ? MOBA_OK : hip_fail(e);
}

size_t moba_dense_workspace_bytes(int dtype, int total_tokens, int total_blocks, int num_heads,
                                  int head_dim, int block_size) {
  if (!dtype_ok(dtype) || total_tokens < 0 || total_blocks < 0 || num_heads < 1 ||
      (head_dim != 64 && head_dim != 128) || block_size < 64 || block_size % 64 != 0)
    return 0;
  return moba::dense_workspace_bytes(dtype == MOBA_BF16, total_blocks, num_heads, head_dim,
                                     block_size);
}

moba_status moba_dense_causal_fwd(const void* q, const void* k, const void* v, int dtype,
                                  const int32_t* cu_seqlens, const int32_t* cu_blocks,
                                  int num_seqs, int total_tokens, int max_seqlen,
                                  int total_blocks, int num_heads, int head_dim,
                                  int block_size, float softmax_scale, void* out,
                                  int out_dtype, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  moba_status st = check_geometry(dtype, cu_seqlens, cu_blocks, num_seqs, total_tokens,
                                  max_seqlen, total_blocks, num_heads, head_dim, block_size);
  if (st != MOBA_OK) return st;
  if (!dtype_ok(out_dtype)) return MOBA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale)) return MOBA_ERR_INVALID_ARG;
  if (total_tokens == 0) return MOBA_OK;
  if (!q || !k || !v || !out || !lse) return MOBA_ERR_INVALID_ARG;
  const bool bf16 = dtype == MOBA_BF16;
  const size_t need = moba::dense_workspace_bytes(bf16, total_blocks, num_heads, head_dim,
                                                  block_size) - kAlign;
  if (need > 0) {
    if (!workspace) return MOBA_ERR_INVALID_ARG;
    if ((uintptr_t)workspace % kAlign != 0) return MOBA_ERR_INVALID_ARG;
    if (workspace_bytes < need) return MOBA_ERR_WORKSPACE_TOO_SMALL;
  }
  moba::Geo g = make_geo(cu_seqlens, cu_blocks, num_seqs, total_tokens, max_seqlen,
                         total_blocks, num_heads, head_dim, block_size);
  hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (bf16) {
    uint16_t* vt = (uint16_t*)workspace;
    uint32_t* vmax = (uint32_t*)((char*)workspace + need - align_up((size_t)num_heads * 4));
    if ((e = timed("v_stage", s, [&] { return moba::launch_v_transpose(v, g, vmax, vt, s); })) !=
        hipSuccess)
      return hip_fail(e);
    if ((e = timed("attn_dense", s, [&] {
           return moba::launch_attn_mfma_dense(q, k, vt, vmax, g, softmax_scale, out,
                                               out_dtype == MOBA_BF16, lse, s);
         })) != hipSuccess)
      return hip_fail(e);
  } else {
    if ((e = timed("attn_dense", s, [&] {
           return moba::launch_attn_f32_dense((const float*)q, (const float*)k,
                                              (const float*)v, g, softmax_scale, out,
                                              out_dtype == MOBA_BF16, lse, s);
         })) != hipSuccess)
      return hip_fail(e);
  }
  return MOBA_OK;
}

moba_status moba_profiler_create(moba_profiler** out) {
  if (!out) return MOBA_ERR_INVALID_ARG;
  *out = new moba_profiler();
  return MOBA_OK;
}

moba_status moba_profiler_attach(moba_profiler* p) {
  g_profiler = p;
  return MOBA_OK;
}

moba_status moba_profiler_reset(moba_profiler* p) {
  if (!p) return MOBA_ERR_INVALID_ARG;
  for (auto& r : p->recs) {
    p->spare.push_back(r.start);
    p->spare.push_back(r.stop);
  }
  p->recs.clear();
  return MOBA_OK;
}

moba_status moba_profiler_read(moba_profiler* p, const char* name, int* launches,
                               double* total_ms) {
  if (!p || !name || !launches || !total_ms) return MOBA_ERR_INVALID_ARG;
  int n = 0;
  double ms = 0.0;
  for (auto& r : p->recs) {
    if (r.name != name) continue;
    hipError_t e = hipEventSynchronize(r.stop);
    if (e != hipSuccess) return hip_fail(e);
    float t = 0.f;
    e = hipEventElapsedTime(&t, r.start, r.stop);
    if (e != hipSuccess) return hip_fail(e);
    ms += t;
    ++n;
  }
  *launches = n;
  *total_ms = ms;
  return MOBA_OK;
}

moba_status moba_profiler_names(moba_profiler* p, char* buf, size_t len) {
  if (!p || !buf || len == 0) return MOBA_ERR_INVALID_ARG;
  std::string all;
  std::vector<std::string> seen;
  for (auto& r : p->recs) {
    bool dup = false;
    for (auto& x : seen) dup = dup || x == r.name;
    if (dup) continue;
    seen.push_back(r.name);
    if (!all.empty()) all += ",";
    all += r.name;
  }
  std::strncpy(buf, all.c_str(), len - 1);
  buf[len - 1] = '\0';
  return MOBA_OK;
}

void moba_profiler_destroy(moba_profiler* p) {
  if (!p) return;
  if (g_profiler == p) g_profiler = nullptr;
  moba_profiler_reset(p);
  for (hipEvent_t e : p->spare) (void)hipEventDestroy(e);
  delete p;
}

}  // extern "C"
