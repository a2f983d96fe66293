/*
 * msa.h -- C ABI of the MI355X (gfx950) MiniMax Sparse Attention library.
 *
 * MiniMax Sparse Attention (MSA) adds, per GQA group, an index branch that
 * scores every earlier key block with one index-query head against one shared
 * index-key head, max-pools the token scores per block and keeps the top-k
 * blocks, always including the query's own (local) block; the main branch
 * then runs exact softmax attention over only those blocks for every head of
 * the group.  Defined on "MiniMax Sparse Attention: let each query pick its
 * own blocks" (ai.thesatyajit.com), section "The mechanism, precisely", and
 * the paper's Figure 1 reproduced there; deployed as block 128, k = 16 (the
 * atlas record of MiniMax M3, atlas.lewiswon.me, summary paragraph).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Sequences are packed token-major ("varlen"): a sequence b has q_len
 *    M_b = cu_seqlens_q[b+1] - cu_seqlens_q[b] query rows and kv_len N_b key
 *    rows.  Its query row t sits at absolute position p = N_b - M_b + t
 *    (bottom-right aligned causal attention): M_b = N_b is a full prefill,
 *    M_b < N_b a chunk of a longer prefill, M_b = 1 a decode step.  Rows with
 *    p < 0 (only when M_b > N_b) attend to nothing: ids -1, output 0, lse -inf.
 *  - Blocks are aligned to absolute position 0: block c holds positions
 *    [c * block_size, (c + 1) * block_size).  The local block is
 *    l = floor(p / block_size).
 *  - topk counts the forced local block: the selection is {l} plus the best
 *    min(topk - 1, l) earlier blocks c < l.  "Best" is the total order
 *    (pooled score descending, block id ascending), so ties go to the lower id
 *    and the result is unique.
 *  - GQA: G = num_kv_heads groups, r = num_heads / G heads per group, query
 *    head h belongs to group floor(h / r).
 *  - All pointers to tensors are device pointers, except where stated.  The
 *    caller owns every buffer and the stream; the library allocates no device
 *    memory and keeps no state between calls.  Every call is asynchronous on
 *    `stream` (0 = the null stream).
 *  - Argument errors are returned before anything is launched.  Values held
 *    in device arrays (sequence lengths, block ids) cannot be checked on the
 *    host: lengths must not exceed max_q_len / max_kv_len and must match the
 *    buffers; the kernels never read outside [row 0, last row of the
 *    sequence], ignore block ids < 0 or > l, and never write outside the rows
 *    the lengths describe.
 *  - Results are deterministic: repeated calls with the same inputs, sizes
 *    and num_splits give bit-identical outputs.  Block ids never depend on
 *    the schedule.  Attention outputs of calls that take different schedules
 *    (another num_splits, or a batch whose size switches between the
 *    KV-outer and the query-outer schedule) agree within bf16 rounding of the
 *    partial results, not bitwise.
 *
 * Supported shapes: block_size 128; head_dim 128; index_dim 64 or 128;
 * 1 <= topk <= 16; num_heads % num_kv_heads == 0 with at most 16 heads per
 * group; 1 <= num_kv_heads <= 16.  Other values return MSA_ERR_UNSUPPORTED.
 * Element types: MSA_F32 (fp32 in, fp32 out) and MSA_BF16 (bf16 in, bf16
 * out); accumulation is fp32 in both.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = 1,  /* null pointer, negative size, bad combination */
  MSA_ERR_UNSUPPORTED = 2,  /* a shape or type the library does not implement */
  MSA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than required */
  MSA_ERR_HIP = 4           /* a HIP launch or runtime call failed */
} msa_status_t;

/* Element types.  MSA_FP8_E4M3 is the OCP 8-bit floating point format E4M3
 * (sign, 4 exponent bits with bias 7, 3 mantissa bits, no infinities; the
 * pages note the kernels also support fp8).  It is accepted for the index
 * tensors of msa_index_topk and, through the *_ex attention calls, for the
 * K/V tensors under bf16 q/out; the plain attention calls (one type for q, K,
 * V and out) return MSA_ERR_UNSUPPORTED for it. */
typedef enum { MSA_F32 = 0, MSA_BF16 = 1, MSA_FP8_E4M3 = 2 } msa_dtype_t;

/* Human-readable name of a status code (static storage, never NULL). */
const char* msa_status_string(msa_status_t status);

/* Last HIP error recorded by a call that returned MSA_ERR_HIP on this host
 * thread (hipSuccess if none). */
int msa_last_hip_error(void);

/* ------------------------------------------------------------------------
 * Index branch: score, block max-pool, top-k with the forced local block.
 *
 * "MiniMax Sparse Attention: let each query pick its own blocks", section
 * "The mechanism, precisely": for query row t and group g the token scores are
 * s_j = q_idx[t, g, :] . k_idx[j, :] (raw dot product, no scale: selection is
 * on raw scores, the "exp-free" top-k of the atlas record's kernel list), the
 * block score is S_c = max over the block's tokens, and the block ids kept are
 * {l} and the best min(topk - 1, l) blocks c < l.  The local block is never
 * scored; every scored block is full.
 *
 *   q_idx        [Tq, G, index_dim]  index queries, Tq = cu_seqlens_q[batch]
 *   k_idx        [Tk, index_dim]     index keys (one head shared by all groups)
 *   dtype        element type of q_idx and k_idx
 *   cu_seqlens_q [batch + 1] int32, device: query row offsets, cu[0] = 0
 *   cu_seqlens_k [batch + 1] int32, device: key row offsets, cu[0] = 0
 *   max_q_len, max_kv_len   host upper bounds of the per-sequence lengths
 *   num_groups   G (= number of KV heads)
 *   block_idx    [Tq, G, topk] int32 out: ascending ids, -1 padded
 *   workspace    device scratch of at least msa_index_topk_workspace_size()
 *                bytes (may be NULL when that size is 0): the fp32 block
 *                scores, batch * max_q_len * G * ceil(max_kv_len / 128) floats
 *                (rounded up to 4 per (row, group)) on the prefill path,
 *                batch * G * ceil(max_kv_len / 128) on the decode path
 *
 * Scores accumulate in fp32.  With max_q_len == 1 (one new token per
 * sequence) the call takes the decode path: the whole index-key cache is
 * streamed once for all groups, then a per-(sequence, group) selection runs.
 * Otherwise the prefill path scans key blocks per query block with an MFMA
 * GEMM whose epilogue max-pools the block scores, then a per-(row, group)
 * selection runs over them.  Both paths use the same total order (score
 * descending, then block id ascending) and return identical ids on identical
 * inputs.
 * ---------------------------------------------------------------------- */
size_t msa_index_topk_workspace_size(int batch, int max_q_len, int max_kv_len, int num_groups,
                                     int block_size, int topk);

msa_status_t msa_index_topk(const void* q_idx, const void* k_idx, msa_dtype_t dtype,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch,
                            int max_q_len, int max_kv_len, int num_groups, int index_dim,
                            int block_size, int topk, int32_t* block_idx, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Main branch, prefill: exact causal softmax attention over the selected
 * blocks, for every head of each group.
 *
 * "MiniMax Sparse Attention: let each query pick its own blocks", section
 * "The mechanism, precisely" (main branch) and the atlas record's summary
 * ("standard scaled dot-product softmax attention"): for head h of group g,
 * J = { j <= p : floor(j / block_size) in Sel(t, g) },
 * z_j = softmax_scale * q[t, h, :] . k[j, g, :], out = softmax(z) V_J,
 * lse = ln sum_j exp(z_j).  There is no sink term.
 *
 *   q            [Tq, num_heads, head_dim]
 *   k, v         [Tk, num_kv_heads, head_dim]
 *   block_idx    [Tq, num_kv_heads, topk] int32 (from msa_index_topk); read
 *                as the set Sel: any order, and -1, ids past the query's
 *                local block and repeated ids add nothing
 *   cu_seqlens_q, cu_seqlens_k, max_q_len, max_kv_len   as for msa_index_topk
 *   softmax_scale  <= 0 selects 1 / sqrt(head_dim)
 *   num_splits   0 = choose the schedule automatically.  For large prefills
 *                (bf16, q_len > 1, at least 4096 (query, group) items) that
 *                is the KV-outer schedule of the atlas record's kernel list:
 *                the selection is inverted into per-block query lists, each
 *                selected K/V block is staged on chip once for every query
 *                that picked it, and the per-block partial results are merged
 *                by a log-sum-exp combine in selection order (no atomics in
 *                any arithmetic).  num_splits >= 1 forces the query-outer
 *                schedule: each selection is split into that many chunks of
 *                consecutive ids, attended separately and merged the same way.
 *   out          [Tq, num_heads, head_dim], element type `dtype`
 *   lse          [Tq, num_heads] fp32, natural log, or NULL
 *   workspace    at least msa_sparse_attn_workspace_size() bytes (the
 *                KV-outer schedule needs about 266 KB per query row of a
 *                window of at most 8192 rows, i.e. up to 2.2 GB)
 * ---------------------------------------------------------------------- */
size_t msa_sparse_attn_workspace_size(int batch, int max_q_len, int max_kv_len, int num_heads,
                                      int num_kv_heads, int head_dim, int topk, int num_splits);

msa_status_t msa_sparse_attn_prefill(const void* q, const void* k, const void* v, msa_dtype_t dtype,
                                     const int32_t* block_idx, const int32_t* cu_seqlens_q,
                                     const int32_t* cu_seqlens_k, int batch, int max_q_len,
                                     int max_kv_len, int num_heads, int num_kv_heads, int head_dim,
                                     int block_size, int topk, float softmax_scale, int num_splits,
                                     void* out, float* lse, void* workspace,
                                     size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Main branch, decode: one new query token per sequence against its cache.
 *
 * Same definition as the prefill call with q_len = 1 and p = ctx_lens[b] - 1
 * (the new token's K/V are already in the cache).  Per the pages
 * ("llama.cpp Merges MiniMax M3's Sparse Attention", key facts) the main
 * branch of a decode step reads about k * block_size = 2,048 tokens
 * regardless of context; the selection is split over num_splits chunks
 * (0 = automatic) so that the block gathers fill the GPU, then combined.
 *
 *   q             [batch, num_heads, head_dim]
 *   k_cache, v_cache  token-major [*, num_kv_heads, head_dim]; sequence b's
 *                 tokens are rows [cache_offsets[b], cache_offsets[b] + ctx_lens[b])
 *   block_idx     [batch, num_kv_heads, topk] int32, read as a set as in the
 *                 prefill call
 *   cache_offsets [batch] int64, device, in tokens
 *   ctx_lens      [batch] int32, device, >= 1, <= max_ctx
 *   out           [batch, num_heads, head_dim]; lse [batch, num_heads] or NULL
 *   workspace     at least msa_sparse_attn_workspace_size(batch, 1, max_ctx, ...) bytes
 * ---------------------------------------------------------------------- */
msa_status_t msa_sparse_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                                    msa_dtype_t dtype, const int32_t* block_idx,
                                    const int64_t* cache_offsets, const int32_t* ctx_lens,
                                    int batch, int max_ctx, int num_heads, int num_kv_heads,
                                    int head_dim, int block_size, int topk, float softmax_scale,
                                    int num_splits, void* out, float* lse, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Main branch with the K/V element type given on its own.
 *
 * The same calls as msa_sparse_attn_prefill / msa_sparse_attn_decode, with
 * `dtype` the element type of q and out and `kv_dtype` that of k and v (the
 * KV cache on the decode path).  Supported pairs: (F32, F32), (BF16, BF16)
 * (exactly the plain calls) and (BF16, FP8_E4M3): an 8-bit KV cache, half
 * the bytes per cached token, for the fp8 support the atlas record of
 * MiniMax M3 notes.  E4M3 K/V elements are widened exactly to bf16 as they
 * are loaded; q.k and P.V then run on the same bf16 MFMAs with fp32
 * accumulation, so an E4M3 K/V tensor gives bit-identical out and lse to
 * the bf16 call on the same values.  There is no scale operand: a per-tensor
 * K scale can be folded into softmax_scale, a V scale applied to out.
 * Other pairs return MSA_ERR_UNSUPPORTED; the workspace size is that of the
 * plain call.
 *
 * block_lse (nullable), [Tq, num_heads, topk] fp32 out: for each selection
 * slot, ln sum over the keys of that slot's block that the row attends of
 * exp(z_j) (z as above), so exp(block_lse - lse) is the share of the head's
 * attention that falls in the block; -inf for a slot that adds no block (-1,
 * a repeat, a block past the local one) and for rows with p < 0.  These are
 * the main branch's block masses the index branch's alignment loss compares
 * against (msa_index_kl_backward).
 * ---------------------------------------------------------------------- */
msa_status_t msa_sparse_attn_prefill_ex(const void* q, const void* k, const void* v, msa_dtype_t dtype,
                                        msa_dtype_t kv_dtype, const int32_t* block_idx,
                                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch,
                                        int max_q_len, int max_kv_len, int num_heads, int num_kv_heads,
                                        int head_dim, int block_size, int topk, float softmax_scale,
                                        int num_splits, void* out, float* lse, float* block_lse,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream);

msa_status_t msa_sparse_attn_decode_ex(const void* q, const void* k_cache, const void* v_cache,
                                       msa_dtype_t dtype, msa_dtype_t kv_dtype, const int32_t* block_idx,
                                       const int64_t* cache_offsets, const int32_t* ctx_lens, int batch,
                                       int max_ctx, int num_heads, int num_kv_heads, int head_dim,
                                       int block_size, int topk, float softmax_scale, int num_splits,
                                       void* out, float* lse, float* block_lse, void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Main branch, backward (prefill layout).
 *
 * The main branch of "MiniMax Sparse Attention: let each query pick its own
 * blocks" ("The mechanism, precisely") is ordinary softmax attention over the
 * keys J of the selected blocks, so its gradients are those of softmax
 * attention restricted to J; the atlas record of MiniMax M3 trains the model
 * through it (the index branch has its own loss and is not differentiated
 * here: block_idx is an input).  With P_j = exp(z_j - lse), delta = dO . out:
 *   dq = scale sum_j P_j (dO . v_j - delta) k_j
 *   dk_j = scale sum over (row, head of the group) of P_j (dO . v_j - delta) q
 *   dv_j = sum over (row, head of the group) of P_j dO
 *
 *   q, k, v, block_idx, cu_seqlens_*, sizes, softmax_scale
 *                as for msa_sparse_attn_prefill (same values as that call)
 *   out, lse     that call's outputs (lse is required)
 *   dout         [Tq, num_heads, head_dim], gradient of out
 *   dtype        MSA_BF16 (q, k, v, out, dout); other types return
 *                MSA_ERR_UNSUPPORTED
 *   dq           [Tq, num_heads, head_dim] fp32 out
 *   dk, dv       [Tk, num_kv_heads, head_dim] fp32 out, overwritten: key rows
 *                no query attends get 0
 *   workspace    at least msa_sparse_attn_backward_workspace_size() bytes:
 *                the per-block edge lists of one window of at most 8192 query
 *                rows, one fp32 per (row, head) and the window's bf16 per-slot
 *                dq contributions (4 KB per (row, group, slot): about 2 GB for
 *                64 query heads, 4 groups and k = 16)
 *
 * Accumulation is fp32; P and dS enter the dK, dV and dQ products as bf16,
 * and each selected block's contribution to dq is kept in bf16 until the
 * fp32 sum over the row's blocks (measured dq error about 2.5e-3 relative RMS).
 * Results are bitwise reproducible (no atomics in any arithmetic: each
 * block's edges are summed in a fixed order).
 * ---------------------------------------------------------------------- */
size_t msa_sparse_attn_backward_workspace_size(int batch, int max_q_len, int max_kv_len, int num_heads,
                                               int num_kv_heads, int head_dim, int topk);

msa_status_t msa_sparse_attn_backward(const void* q, const void* k, const void* v, const void* out,
                                      const void* dout, const float* lse, msa_dtype_t dtype,
                                      const int32_t* block_idx, const int32_t* cu_seqlens_q,
                                      const int32_t* cu_seqlens_k, int batch, int max_q_len, int max_kv_len,
                                      int num_heads, int num_kv_heads, int head_dim, int block_size, int topk,
                                      float softmax_scale, float* dq, float* dk, float* dv, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Index branch, KL alignment loss and its gradients.
 *
 * "MiniMax Sparse Attention: let each query pick its own blocks", section
 * "Two design choices": an auxiliary KL loss aligns the index branch's block
 * scores with the main attention's distribution over blocks, behind a
 * stop-gradient so that only the index projections learn; the atlas record
 * of MiniMax M3 (summary) takes the group-averaged main-branch distribution
 * as the target.  For query row t and group g, over the attended slots i of
 * its selection (Sel read as a set) with c_i the slot's block:
 *   A_i = mean over the group's heads h of exp(block_lse[t, h, i] - lse[t, h])
 *   S_i = max over the keys j <= p of block c_i of q_idx[t, g] . k_idx[j]
 *         (raw dot product in fp32; j*_i = the lowest such key reaching it)
 *   loss[t, g] = sum_i A_i (ln A_i - ln softmax_i(S))    (0 for rows p < 0)
 * A is a constant target: no gradient reaches the main branch.  With respect
 * to the sum of loss over all rows and groups, dS_i = softmax_i(S) sum_k A_k
 * - A_i, passed through the max to the argmax key:
 *   dq_idx[t, g] = sum_i dS_i k_idx[j*_i],  dk_idx[j*_i] += dS_i q_idx[t, g].
 *
 *   q_idx, k_idx, dtype     as for msa_index_topk (fp32 or bf16)
 *   block_idx               the selection both calls used
 *   lse, block_lse          [Tq, num_heads] and [Tq, num_heads, topk] fp32 from
 *                           msa_sparse_attn_prefill_ex on the same selection
 *   loss                    [Tq, num_groups] fp32 out
 *   dq_idx                  [Tq, num_groups, index_dim] fp32 out
 *   dk_idx                  [Tk, index_dim] fp32 out, overwritten (0 for keys
 *                           that are no argmax)
 *   workspace               at least msa_index_kl_workspace_size() bytes
 * Results are bitwise reproducible (each block's edges are summed in a fixed
 * order).  Other element types return MSA_ERR_UNSUPPORTED.
 * ---------------------------------------------------------------------- */
size_t msa_index_kl_workspace_size(int batch, int max_q_len, int max_kv_len, int num_groups, int topk);

msa_status_t msa_index_kl_backward(const void* q_idx, const void* k_idx, msa_dtype_t dtype,
                                   const int32_t* block_idx, const float* lse, const float* block_lse,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch,
                                   int max_q_len, int max_kv_len, int num_heads, int num_groups, int index_dim,
                                   int block_size, int topk, float* loss, float* dq_idx, float* dk_idx,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ----------------------------------------------------------------------
 * Index front-end: hidden states -> index-query heads and index-key head.
 *
 * "MiniMax Sparse Attention: let each query pick its own blocks", Figure 1:
 * the index branch passes the hidden states through a linear projection, a
 * norm and RoPE before the score matrix.  The atlas record of MiniMax M3
 * (provenance notes on section 5.1) gives the model width (3072) and a rotary
 * width of 64 of the 128 head dims for the main heads; the pages name neither
 * the norm's kind nor the rotary base.  This call computes, per token and per
 * head vector (G query heads, then the key head):
 *   y   = W_h x                               (no bias)
 *   y_i = gain_i * y_i / sqrt(mean_i y_i^2 + norm_eps)   (RMS norm per head)
 *   for i < rope_dim/2, the pair (y_i, y_{i + rope_dim/2}) turned by the angle
 *   p * rope_theta^(-2i/rope_dim): (a, b) -> (a cos - b sin, b cos + a sin);
 *   dims >= rope_dim are left as they are.
 * p is the token's absolute position, p = N - M + t for token t of a sequence
 * with q_len M and kv_len N (the convention of the other calls).
 *
 *   x                     [total_q, d_model] hidden states of the new tokens,
 *                         packed by cu_seqlens_q (dtype fp32 or bf16)
 *   w_q                   [num_groups * index_dim, d_model]: rows g*index_dim ..
 *                         (g+1)*index_dim-1 project to the query head of group g
 *   w_k                   [index_dim, d_model]: the shared key head
 *   q_norm_weight         [index_dim] fp32 gain of the query heads' norm
 *   k_norm_weight         [index_dim] fp32 gain of the key head's norm
 *   cu_seqlens_q/_k       device [batch+1] int32; cu_seqlens_q[batch] must equal
 *                         total_q
 *   q_idx                 out [total_q, num_groups, index_dim] (out_dtype)
 *   k_idx                 out: the index-key rows of the new tokens, written at
 *                         row cu_seqlens_k[b] + p (the caller's index-key cache
 *                         laid out as msa_index_topk reads it: in a decode step
 *                         with M = 1 this appends the new token's key at
 *                         position N - 1; rows of other positions are not
 *                         touched; a token with p < 0 writes no key row)
 *   out_dtype             fp32 or bf16 (the type msa_index_topk then reads)
 * Sizes: index_dim 64 or 128, d_model a multiple of 64, rope_dim 0, 64 or (for
 * index_dim 128) 128; others return MSA_ERR_UNSUPPORTED.  fp32 accumulation;
 * the angle is reduced in fp64.  No workspace; deterministic.  With total_q 0,
 * x, q_idx and k_idx may be null and nothing is launched.
 * ---------------------------------------------------------------------- */
msa_status_t msa_index_frontend(const void* x, const void* w_q, const void* w_k, msa_dtype_t dtype,
                                const float* q_norm_weight, const float* k_norm_weight,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch,
                                int64_t total_q, int d_model, int num_groups, int index_dim, int rope_dim,
                                float rope_theta, float norm_eps, void* q_idx, void* k_idx,
                                msa_dtype_t out_dtype, hipStream_t stream);

/* ----------------------------------------------------------------------
 * Index front-end backward: gradients of the front-end's parameters.
 *
 * The alignment loss trains only the index branch: the atlas record of
 * MiniMax M3 (summary paragraph) confines it to the index projections by a
 * stop-gradient on the indexer's input, so x is held constant and no dx is
 * produced.  For upstream gradients dq_idx (of q_idx) and dk_idx (of the
 * index-key rows, e.g. those of msa_index_kl_backward), per token and head
 * vector, with n = y / r, r = sqrt(mean y^2 + norm_eps), z = gain * n and
 * out = R z (R the rotation of msa_index_frontend):
 *   dz = R^T dout,  dgain += dz * n,  dn = dz * gain,
 *   dy = (dn - n (dn . n) / index_dim) / r,  dW_h += dy x^T.
 *
 *   x, w_q, w_k, norm weights, cu_seqlens, sizes, rope_dim, rope_theta,
 *   norm_eps               as for msa_index_frontend (bf16 x and weights only)
 *   dq_idx                 [total_q, num_groups, index_dim] fp32
 *   dk_idx                 fp32 index-key gradient rows; the row of token t of
 *                          sequence b is cu_seqlens_k[b] + p (rows of other
 *                          positions are not read; tokens with p < 0 or
 *                          p >= kv_len have no key row and contribute nothing
 *                          through the key head)
 *   dw_q, dw_k             out [num_groups * index_dim, d_model] and
 *                          [index_dim, d_model] fp32, overwritten
 *   dq_norm_weight,
 *   dk_norm_weight         out [index_dim] fp32, overwritten
 *   workspace              at least msa_index_frontend_backward_workspace_size()
 *                          bytes: dy in bf16 per (token, projection row), fp32
 *                          weight-gradient slices of the token ranges, and
 *                          per-workgroup gain partials (about 240 MB for
 *                          128K tokens at d_model 3072)
 * The weight gradient is accumulated in fp32 from bf16 dy and x on MFMAs;
 * slices and partials are summed in a fixed order, so results are bitwise
 * reproducible.  fp32 inputs return MSA_ERR_UNSUPPORTED.  With total_q 0, x,
 * dq_idx and dk_idx may be null and the outputs are set to zero.
 * ---------------------------------------------------------------------- */
size_t msa_index_frontend_backward_workspace_size(int64_t total_q, int d_model, int num_groups, int index_dim);

msa_status_t msa_index_frontend_backward(const void* x, const void* w_q, const void* w_k, msa_dtype_t dtype,
                                         const float* q_norm_weight, const float* k_norm_weight,
                                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch,
                                         int64_t total_q, int d_model, int num_groups, int index_dim, int rope_dim,
                                         float rope_theta, float norm_eps, const float* dq_idx, const float* dk_idx,
                                         float* dw_q, float* dw_k, float* dq_norm_weight, float* dk_norm_weight,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * msa_index_topk without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation.  Same arguments, checks, kernels and results as
 * msa_index_topk (bit-identical block ids), minus the workspace: the scratch
 * is a static device array of MSA_NOALLOC_SCRATCH_BYTES inside the library,
 * one per GPU, held until the process ends.  Calls whose
 * msa_index_topk_workspace_size() exceeds it return MSA_ERR_WORKSPACE before
 * any launch (for example decode of 32 sequences at 1M context needs 4 MiB;
 * prefill needs rows * G * ceil(max_kv_len / 128) * 4 bytes).  `stream` must
 * belong to the current device (MSA_ERR_INVALID_ARG otherwise).  The call
 * allocates nothing (no hipMalloc, no memset) and keeps no result in the
 * scratch that a later call relies on.  All calls on one GPU share its
 * scratch: calls that may overlap in time on one GPU (different streams
 * without ordering, several host threads) race and give undefined ids;
 * serialize them on one stream.
 * ---------------------------------------------------------------------- */
#define MSA_NOALLOC_SCRATCH_BYTES (32u << 20)

msa_status_t msa_index_topk_noalloc(const void* q_idx, const void* k_idx, msa_dtype_t dtype,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int batch,
                                    int max_q_len, int max_kv_len, int num_groups, int index_dim,
                                    int block_size, int topk, int32_t* block_idx, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MSA_H */
