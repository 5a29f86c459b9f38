/*
 * moba.h - C ABI of libmoba.so: MoBA (Mixture of Block Attention) causal
 * prefill forward on AMD Instinct MI355X (gfx950).
 *
 * The operation (cited by page title and section):
 *   "MoBA: Learned Block Sparsity for Long-Context Attention" (wispaper.ai
 *   review), section "The Change: Treat KV Blocks as Experts and Route Queries
 *   with Top-k Gating": K/V are split into blocks of B tokens, each block's
 *   keys are mean-pooled, a query scores each block by its inner product with
 *   the pooled key, keeps the top-k blocks, never selects a future block,
 *   always selects its own block (with a causal mask inside it), and runs
 *   exact softmax attention over the selected blocks' tokens.  Section
 *   "Efficiency and Implementation" (Algorithm 1): queries are arranged by the
 *   KV blocks they selected, own-block and historical-block attention are
 *   computed separately and combined with an online softmax.
 *
 * Conventions shared by every call
 *   - Tensors are dense row-major and live in device memory owned by the
 *     caller: q, k, v, out are [total_tokens, num_heads, head_dim]; lse is
 *     [total_tokens, num_heads]; kbar is [total_blocks, num_heads, head_dim];
 *     block_idx is [total_tokens, num_heads, topk].
 *   - Variable-length batches are packed: sequence s owns tokens
 *     [cu_seqlens[s], cu_seqlens[s+1]) and blocks [cu_blocks[s],
 *     cu_blocks[s+1]) with cu_blocks[s+1] - cu_blocks[s] = ceil(L_s / B).
 *     Blocks never cross sequences; block ids inside block_idx are local to
 *     the sequence and 0-based.  The last block of a sequence may be partial.
 *     cu_seqlens and cu_blocks are device int32 arrays of num_seqs + 1
 *     entries.  The host passes the matching scalars (total_tokens,
 *     max_seqlen = max L_s, total_blocks = cu_blocks[num_seqs]) so that no
 *     call reads device memory from the host; they must agree with the
 *     arrays (the kernels clamp every index, so a mismatch gives wrong
 *     numbers, not out-of-bounds accesses of q/k/v).
 *   - dtype (moba_dtype) is the element type of q, k, v: MOBA_BF16 (the
 *     production path: bf16 MFMA, fp32 accumulation) or MOBA_F32 (fp32 VALU
 *     path for small, high-precision checks).
 *   - Supported: head_dim 64 or 128; block_size a positive multiple of 64;
 *     1 <= topk <= 64; total_tokens * topk < 2^31.  The query lists of the
 *     attention calls hold 32-bit offsets, so moba_attn_fwd also needs
 *     total_tokens * heads per pass * (topk - 1) < 2^31 (see head_chunk) and
 *     moba_attn_bwd total_tokens * num_heads * (topk - 1) < 2^31; a larger
 *     geometry returns MOBA_ERR_UNSUPPORTED before anything is launched.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL is the
 *     default stream), allocates no device memory and keeps no state between
 *     calls.  Arguments are validated on the host before anything is
 *     launched; an invalid call launches nothing and returns an error.
 *   - Errors: MOBA_OK (0) or a negative moba_status.  MOBA_ERR_HIP means a
 *     launch failed; moba_last_hip_error() returns that HIP error code
 *     (per calling thread).  The library never prints or aborts.
 */
#ifndef MOBA_H_
#define MOBA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOBA_API_VERSION 6

/* Size of the device workspace moba_attn_fwd_static keeps inside the library
 * (per GPU, for the life of the process). */
#define MOBA_STATIC_WORKSPACE_BYTES (256u << 20)

typedef enum moba_status {
  MOBA_OK = 0,
  MOBA_ERR_INVALID_ARG = -1,         /* null pointer, negative size, inconsistent geometry */
  MOBA_ERR_UNSUPPORTED = -2,         /* valid but outside the supported shapes or dtypes */
  MOBA_ERR_WORKSPACE_TOO_SMALL = -3, /* workspace_bytes below the required size */
  MOBA_ERR_HIP = -4                  /* a HIP launch failed, see moba_last_hip_error() */
} moba_status;

typedef enum moba_dtype {
  MOBA_F32 = 0,
  MOBA_BF16 = 1
} moba_dtype;

/* ABI version of the loaded library (its MOBA_API_VERSION). */
int moba_api_version(void);

/* Human-readable name of a moba_status; never NULL. */
const char* moba_status_str(int status);

/* HIP error code (hipError_t as int) of the last MOBA_ERR_HIP on this thread. */
int moba_last_hip_error(void);

/*
 * Block mean-pool of the keys.
 *   kbar[b, h, :] = mean of k[t, h, :] over the tokens t of block b (a partial
 *   last block averages the tokens it has).
 * Defined by the mean_pool(K[I_i]) of the affinity in "MoBA: Learned Block
 * Sparsity for Long-Context Attention", section "The Change", and step 2 of
 * "MoBA: 面向长上下文大语言模型的混合块注意力机制" (技术实现).
 *   k      [total_tokens, num_heads, head_dim], dtype
 *   kbar   [total_blocks, num_heads, head_dim] fp32, written in full
 *   kbar3  bf16 bit patterns, total_blocks * num_heads * 3 * head_dim of
 *          them, or NULL (not written): the same means as an exact sum of
 *          three bf16 terms, kbar = hi + mid + lo, where hi is the upper half
 *          of kbar's fp32 pattern, mid the upper half of kbar - hi and lo the
 *          (exactly representable) rest.  Layout [num_heads][3 terms]
 *          [head_dim / 16][total_blocks][16]: term x of element e of block b,
 *          head h sits at ((h * 3 + x) * (head_dim / 16) + e / 16) *
 *          total_blocks * 16 + b * 16 + e % 16.  This is the form in which
 *          the bf16 gate reads the pooled keys: three exact bf16 products per
 *          element on the matrix cores give the fp32 score, and one load
 *          reads the k-step fragments of 32 consecutive blocks at once.
 *          (Exact for means of magnitude 2^-110 or more.)
 * Summation is fp32 in a fixed order (deterministic).
 */
moba_status moba_pool_keys(const void* k, int dtype,
                           const int32_t* cu_seqlens, const int32_t* cu_blocks,
                           int num_seqs, int total_tokens, int max_seqlen,
                           int total_blocks, int num_heads, int head_dim,
                           int block_size, float* kbar, uint16_t* kbar3, void* stream);

/*
 * Gate and causal top-k selection.
 * For query token t (local position p, own block c = p / B) and head h:
 *   s_i = <q[t, h, :], kbar[block i, h, :]> for past blocks i < c only
 *   (future blocks are masked out of routing); the own block c is always
 *   selected and counts toward topk; the remaining topk - 1 slots take the
 *   highest s_i, ties going to the lower block index; rows with c < topk - 1
 *   select every block 0..c.
 * "MoBA: Learned Block Sparsity for Long-Context Attention", section "The
 * Change" (affinity, hard top-k gate, causality rules).
 *   q          [total_tokens, num_heads, head_dim], dtype
 *   kbar       output of moba_pool_keys; read for fp32 queries
 *   kbar3      its three-term bf16 form from moba_pool_keys; read for bf16
 *              queries (required then; may be NULL for fp32)
 *   block_idx  [total_tokens, num_heads, topk] int32, written in full: the
 *              selected local block ids in ascending order (so the own block
 *              is the last valid entry), then -1 padding
 * Scores are fp32 (fp32 products of the exact inputs, fp32 accumulation).
 */
moba_status moba_gate_topk(const void* q, int dtype, const float* kbar,
                           const uint16_t* kbar3, const int32_t* cu_seqlens,
                           const int32_t* cu_blocks,
                           int num_seqs, int total_tokens, int max_seqlen,
                           int total_blocks, int num_heads, int head_dim,
                           int block_size, int topk, int32_t* block_idx,
                           void* stream);

/*
 * Min/max pooling of the keys (the pooled representation of the min/max
 * gate below).  "MoBA: Mixture of Block Attention for Long-Context LLMs"
 * (research.elamur.ai), "Key points": Quest reads as MoBA with smaller blocks
 * and min/max pooling.
 *   kmax[b, h, :] = elementwise max of k[t, h, :] over the tokens t of
 *   block b;  kmin[b, h, :] = elementwise min.  Exact (no rounding).
 *   k        [total_tokens, num_heads, head_dim], dtype
 *   kminmax  num_heads * total_blocks * 2 * head_dim fp32, written in full,
 *            group-major: with r = [kmax[b, h, :], kmin[b, h, :]] (2 head_dim
 *            values) and G = head_dim / 2 groups of 4 per row,
 *            kminmax[((h * G + g) * total_blocks + b) * 4 + i] = r[4 g + i],
 *            i.e. a [num_heads, G, total_blocks, 4] array, so that the gate
 *            reads one group of consecutive blocks as one contiguous run
 */
moba_status moba_pool_minmax(const void* k, int dtype, const int32_t* cu_seqlens,
                             const int32_t* cu_blocks, int num_seqs, int total_tokens,
                             int max_seqlen, int total_blocks, int num_heads, int head_dim,
                             int block_size, float* kminmax, void* stream);

/*
 * Gate and causal top-k with the min/max pooled score.  As moba_gate_topk
 * (same causality, forced own block counted in topk, ties to the lower
 * block index, same block_idx format) with the score of past block i
 *   s_i = sum_e max(q_e * kmin_i[e], q_e * kmax_i[e])
 *       = the largest q . x over the box [kmin_i, kmax_i] of block i,
 * an upper bound of q . k for every key k of the block (the reading of
 * min/max pooling adopted here; the page gives no formula).
 *   kminmax  output of moba_pool_minmax
 * bf16 inputs only (MOBA_ERR_UNSUPPORTED for MOBA_F32).  Products are exact,
 * accumulation fp32.
 */
moba_status moba_gate_topk_minmax(const void* q, int dtype, const float* kminmax,
                                  const int32_t* cu_seqlens, const int32_t* cu_blocks,
                                  int num_seqs, int total_tokens, int max_seqlen,
                                  int total_blocks, int num_heads, int head_dim, int block_size,
                                  int topk, int32_t* block_idx, void* stream);

/*
 * Static routing: a fixed gate in place of moba_gate_topk.
 * "MoBA: Learned Block Sparsity for Long-Context Attention", section "Why
 * the Change Is Plausible" (static sparse patterns as special cases of the
 * gate: sliding-window attention always routes to the most recent blocks,
 * attention-sink attention to the initial blocks plus the recent ones, full
 * attention is k = n).  With the same causality as the learned gate, the row
 * of a query whose own block is c holds
 *   every block 0..c                                  when c < topk, else
 *   blocks 0..s-1 and c-(topk-1-s)..c, s = min(sink_blocks, topk - 1),
 * ascending, then -1 padding.  sink_blocks = 0 is a sliding window of topk
 * blocks (own included); topk >= the longest sequence's block count is full
 * causal attention.  The rows are the same for every head.
 *   block_idx   [total_tokens, num_heads, topk] int32, written in full, in
 *               the format of moba_gate_topk (input of moba_attn_fwd)
 *   sink_blocks >= 0 (MOBA_ERR_INVALID_ARG otherwise)
 * Geometry arguments as for the other calls (block_size a multiple of 64).
 */
moba_status moba_static_select(const int32_t* cu_seqlens, const int32_t* cu_blocks,
                               int num_seqs, int total_tokens, int max_seqlen,
                               int total_blocks, int num_heads, int block_size, int topk,
                               int sink_blocks, int32_t* block_idx, void* stream);

/*
 * Workspace bytes moba_attn_fwd needs for this geometry and head_chunk (0
 * when the arguments are invalid).  The workspace holds, for the heads of one
 * pass, the per-(KV block, head) query lists, the per-(query, selected block)
 * partial results and a transposed copy of V, so it scales with head_chunk:
 * about total_tokens * heads per pass * topk * (2 head_dim + 8) bytes.
 *   head_chunk  heads per pass of moba_attn_fwd; 0, or any value of at least
 *               num_heads, means all heads in one pass; negative is invalid
 */
size_t moba_attn_workspace_bytes(int dtype, int total_tokens, int total_blocks,
                                 int num_heads, int head_dim, int block_size,
                                 int topk, int head_chunk);

/*
 * Sparse attention over the selected blocks.
 *   out[t, h, :] = sum_{j in J} softmax_j(scale * <q[t,h], k[j,h]>) v[j, h, :]
 *   lse[t, h]    = ln sum_{j in J} exp(scale * <q[t,h], k[j,h]>)
 * where J is the union of the tokens of the historical blocks listed in
 * block_idx[t, h, :] and the own-block tokens up to and including t.
 * "Mixture of Block Attention (MoBA)" (globaladvisors.biz), "Underlying
 * computational mechanism" (Softmax(q K[I]^T) V[I]); "MoBA: Learned Block
 * Sparsity for Long-Context Attention", "Efficiency and Implementation"
 * (queries arranged per KV block, own-block and historical attention
 * computed separately, merged with an online softmax).
 *   block_idx  as written by moba_gate_topk (or any caller-made selection in
 *              the same format: ascending, then -1).  Entries that are
 *              negative, not below the own block, or not increasing are
 *              ignored, as is any historical entry after the first
 *              topk - 1; the own block is always attended.
 *   out        [total_tokens, num_heads, head_dim], out_dtype (F32 or BF16)
 *   lse        [total_tokens, num_heads] fp32, natural log
 *   head_chunk heads per pass (0 or >= num_heads: all heads at once).  The
 *              heads are processed in consecutive groups of head_chunk, one
 *              after the other on `stream`, each group reusing the same
 *              workspace; the results do not depend on head_chunk.  Heads
 *              are independent in MoBA, which is what lets a layer too large
 *              for one workspace run head group by head group ("MoBA:
 *              Learned Block Sparsity for Long-Context Attention",
 *              "Efficiency and Implementation": the 10M-token run splits the
 *              work at the level of query heads).
 *   workspace  device buffer of at least moba_attn_workspace_bytes(...,
 *              head_chunk) bytes, 256-byte aligned; its contents on entry
 *              are ignored
 * Results are bitwise reproducible: no floating-point atomics, and each
 * query's arithmetic depends only on its own data and its selected blocks,
 * not on the (scheduling-dependent) order of the query lists.
 */
moba_status moba_attn_fwd(const void* q, const void* k, const void* v, int dtype,
                          const int32_t* cu_seqlens, const int32_t* cu_blocks,
                          int num_seqs, int total_tokens, int max_seqlen,
                          int total_blocks, int num_heads, int head_dim,
                          int block_size, int topk, const int32_t* block_idx,
                          float softmax_scale, void* out, int out_dtype,
                          float* lse, int head_chunk, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * moba_attn_fwd for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and results, with the workspace taken from a fixed
 * device array inside the library instead of a caller buffer.  The array
 * holds MOBA_STATIC_WORKSPACE_BYTES (256 MiB) on each GPU the library runs
 * on, from the first call on that GPU until the process ends; the call
 * itself allocates nothing.
 *   Arguments as for moba_attn_fwd, without head_chunk and the workspace.
 *   The heads run in passes of as many heads as fit in the array
 *   (moba_attn_workspace_bytes(..., head_chunk) <= MOBA_STATIC_WORKSPACE_BYTES);
 *   when not even one head fits (about total_tokens * topk * (2 head_dim + 8)
 *   bytes per head, e.g. 32K tokens at topk 32 and head_dim 128), the call
 *   returns MOBA_ERR_WORKSPACE_TOO_SMALL and launches nothing.
 *   Every call on one GPU uses that GPU's one array, and the array keeps the
 *   last call's contents (every piece a call reads is written or cleared by
 *   that call first).  Calls that overlap on one GPU (on different streams,
 *   or from several threads without ordering) race on the array and give
 *   wrong results: serialise them.
 */
moba_status moba_attn_fwd_static(const void* q, const void* k, const void* v, int dtype,
                                 const int32_t* cu_seqlens, const int32_t* cu_blocks,
                                 int num_seqs, int total_tokens, int max_seqlen,
                                 int total_blocks, int num_heads, int head_dim,
                                 int block_size, int topk, const int32_t* block_idx,
                                 float softmax_scale, void* out, int out_dtype, float* lse,
                                 void* stream);

/*
 * Backward of moba_attn_fwd: gradients of out with respect to q, k and v for
 * the selections in block_idx.  The block selection is a hard top-k and is
 * not differentiated; gradients flow through the softmax attention over each
 * query's selected tokens ("MoBA: Learned Block Sparsity for Long-Context
 * Attention", "The Change": MoBA trains end to end as a drop-in for full
 * attention; "MoBA: Mixture of Block Attention for Long-Context LLMs"
 * (research.elamur.ai), "Key points").  With P[t, j] = exp(scale q_t.k_j -
 * lse[t]) over the attended pairs and D[t] = dout[t] . out[t]:
 *   dv[j] = sum_t P[t, j] dout[t]
 *   dS[t, j] = P[t, j] (dout[t] . v[j] - D[t])
 *   dq[t] = scale sum_j dS[t, j] k[j],   dk[j] = scale sum_t dS[t, j] q[t]
 * (per head; sums over the attended pairs only).
 *   q, k, v      the forward's inputs, bf16 only (MOBA_ERR_UNSUPPORTED else)
 *   out, lse     the forward's outputs for the same inputs, selections and
 *                scale (out in out_dtype, F32 or BF16; lse fp32)
 *   dout         [total_tokens, num_heads, head_dim] bf16, upstream gradient
 *   block_idx    the selections the forward used
 *   dq, dk, dv   [total_tokens, num_heads, head_dim] fp32, written in full
 *   workspace    at least moba_attn_bwd_workspace_bytes(...) bytes, 256-byte
 *                aligned; contents on entry ignored
 * dk and dv take no atomics, but each key's sums run over its block's query
 * list, whose order depends on scheduling; dq is summed with fp32 atomics
 * over the query's (at most topk) selected blocks.  The last bits of all
 * three may therefore vary between runs (the forward's do not).
 */
size_t moba_attn_bwd_workspace_bytes(int dtype, int total_tokens, int total_blocks,
                                     int num_heads, int head_dim, int block_size, int topk);

moba_status moba_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                          int out_dtype, const void* dout, const float* lse, int dtype,
                          const int32_t* cu_seqlens, const int32_t* cu_blocks, int num_seqs,
                          int total_tokens, int max_seqlen, int total_blocks, int num_heads,
                          int head_dim, int block_size, int topk, const int32_t* block_idx,
                          float softmax_scale, float* dq, float* dk, float* dv, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Workspace bytes moba_dense_causal_fwd needs (0 when arguments are invalid). */
size_t moba_dense_workspace_bytes(int dtype, int total_tokens, int total_blocks,
                                  int num_heads, int head_dim, int block_size);

/*
 * Dense causal softmax attention (the exact baseline MoBA is compared with:
 * "MoBA: Learned Block Sparsity for Long-Context Attention", section
 * "Starting Point: Exact Softmax Attention and Its Cost").
 *   out[t, h, :] and lse[t, h] as in moba_attn_fwd with J = every token of
 *   t's sequence up to and including t.
 * The block geometry (block_size, cu_blocks, total_blocks) only lays out the
 * transposed-V staging copy in the workspace; any multiple of 64 works.
 */
moba_status moba_dense_causal_fwd(const void* q, const void* k, const void* v, int dtype,
                                  const int32_t* cu_seqlens, const int32_t* cu_blocks,
                                  int num_seqs, int total_tokens, int max_seqlen,
                                  int total_blocks, int num_heads, int head_dim,
                                  int block_size, float softmax_scale, void* out,
                                  int out_dtype, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * Measurement support (not part of the computation): sustained bf16 MFMA
 * rate probes.  Launches `workgroups` workgroups of 4 waves; every wave runs
 * 4 independent chains of `iterations` v_mfma_f32_32x32x16_bf16, i.e.
 * workgroups * 4 * 4 * iterations * 32768 flops.  `operands` selects the
 * data the products see:
 *   0  one fixed, low-entropy operand pair in registers (no memory traffic)
 *   1  random bf16 operands cycling through eight register sets
 *   2  random register A operands and a random B operand read from LDS for
 *      every product (1 KiB per wave per MFMA)
 * The caller times it (events on `stream`) to obtain the rate the chip
 * sustains at the clock it holds under that load.
 *   sink  device buffer of at least workgroups * 256 floats (written; the
 *         values only keep the products from being optimised away)
 * Returns MOBA_ERR_INVALID_ARG for workgroups or iterations below 1, a null
 * sink, operands outside 0..2, or iterations not a multiple of 8 with
 * operands 1 or 2.
 */
moba_status moba_probe_mfma_rate(int workgroups, int iterations, int operands, float* sink,
                                 void* stream);

/*
 * Measurement support (not part of the computation).
 * A profiler attached to the calling thread brackets every kernel launch the
 * library makes from that thread with a pair of HIP events on the launch's
 * stream and accumulates, per kernel name, the number of launches and their
 * total duration.  The profiler owns its events (host-side HIP objects; no
 * device memory); the results of the computation do not depend on it.
 *   moba_profiler_create   returns a new profiler in *out
 *   moba_profiler_attach   attaches p to the calling thread (NULL detaches)
 *   moba_profiler_reset    forgets all recorded launches
 *   moba_profiler_read     waits for the recorded events and returns the
 *                          launches and total milliseconds of kernel `name`
 *                          (0 and 0.0 if it never ran); names are the
 *                          kernels' short names, e.g. "attn_hist"
 *   moba_profiler_names    writes the distinct kernel names seen so far as a
 *                          comma-separated list into buf (truncated to len)
 *   moba_profiler_destroy  frees p (detach it first)
 */
typedef struct moba_profiler moba_profiler;
moba_status moba_profiler_create(moba_profiler** out);
moba_status moba_profiler_attach(moba_profiler* p);
moba_status moba_profiler_reset(moba_profiler* p);
moba_status moba_profiler_read(moba_profiler* p, const char* name, int* launches,
                               double* total_ms);
moba_status moba_profiler_names(moba_profiler* p, char* buf, size_t len);
void moba_profiler_destroy(moba_profiler* p);

#ifdef __cplusplus
}
#endif

#endif /* MOBA_H_ */
