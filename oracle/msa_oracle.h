/*
 * msa_oracle.h -- plain CPU oracle for MiniMax Sparse Attention (MSA).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link or
 * call this.  It is the slow, obviously correct definition that the GPU path
 * is checked against; it shares no code, header or constant with the GPU
 * library.
 *
 * What it computes (sources, by page title and section):
 *   - "MiniMax Sparse Attention: let each query pick its own blocks"
 *     (ai.thesatyajit.com), section "The mechanism, precisely", and the
 *     paper's Figure 1 reproduced there: per GQA group one index-query head is
 *     dotted with one shared index-key head, the token scores are max-pooled
 *     into fixed key blocks, the top-k blocks are kept, the query's own
 *     (local) block is always kept, and the main branch runs exact softmax
 *     attention over the kept blocks for every head of the group.
 *   - The atlas record of MiniMax M3 (atlas.lewiswon.me), summary paragraph:
 *     standard scaled dot-product softmax attention; selection on raw
 *     max-pooled dot products; block 128, k = 16, local block forced in.
 *
 * Conventions (readings where the pages are silent):
 *   - k counts the forced local block: Sel = {local} + best (k-1) earlier blocks.
 *   - Order for selection: block score descending, then block id ascending.
 *   - Blocks are aligned to absolute position 0.  Query row t of a sequence
 *     with q_len M and kv_len N sits at position p = N - M + t.
 *   - Index scores: raw dot product accumulated in fp32, sequentially over d.
 *   - Attention: fp64 throughout, natural-log LSE, no sink term.
 *
 * Element type codes for inputs: 0 = fp32, 1 = bf16 bit patterns (uint16),
 * widened exactly to fp32 by a 16-bit left shift, 2 = 8-bit floating point
 * E4M3 bit patterns (uint8) as the OCP 8-bit floating point specification
 * defines them (sign, 4 exponent bits with bias 7, 3 mantissa bits,
 * subnormals at exponent 0, no infinities, S.1111.111 is NaN), decoded
 * exactly.  The pages note fp8 support in the kernels; code 2 is used for
 * the index tensors and for an 8-bit KV cache.
 */
#ifndef MSA_ORACLE_H
#define MSA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Block selection for n query rows.
 *   q_idx  : [n][G][DI]        index queries of the n rows (compact)
 *   k_idx  : [*][DI]           index keys; row r's sequence starts at kstart[r]
 *   pos    : [n]               absolute position p of each row (p < 0: no keys)
 *   sel    : [n][G][topk] out  ascending block ids, -1 padded
 *   scores : [n][G][nbmax] out (nullable) pooled block scores for c < p/Bk,
 *            -inf elsewhere; nbmax is the caller's row stride.
 * Returns 0 on success, nonzero on bad arguments. */
int oracle_index_topk(const void* q_idx, const void* k_idx, int dtype,
                      const int64_t* kstart, const int64_t* pos, int64_t n,
                      int G, int DI, int Bk, int topk, int32_t* sel,
                      float* scores, int64_t nbmax);

/* Exact sparse attention for n query rows.
 *   q    : [n][Hq][D]          queries of the n rows (compact)
 *   k, v : [*][Hkv][D]         keys / values; row r's sequence starts at kstart[r]
 *   sel  : [n][Hkv][topk]      selected block ids (entries < 0 ignored)
 *   out  : [n][Hq][D]  fp64 out
 *   lse  : [n][Hq]     fp64 out (natural log; -inf when no key is attended)
 * Head h uses KV head / group h / (Hq / Hkv). */
int oracle_sparse_attn(const void* q, const void* k, const void* v, int dtype,
                       const int64_t* kstart, const int64_t* pos, const int32_t* sel,
                       int64_t n, int Hq, int Hkv, int D, int Bk, int topk,
                       double scale, double* out, double* lse);

/* As oracle_sparse_attn with q read as `dtype` and k, v as `kv_dtype` (an
 * 8-bit KV cache under bf16 queries: dtype 1, kv_dtype 2). */
int oracle_sparse_attn_kv(const void* q, const void* k, const void* v, int dtype, int kv_dtype,
                          const int64_t* kstart, const int64_t* pos, const int32_t* sel,
                          int64_t n, int Hq, int Hkv, int D, int Bk, int topk,
                          double scale, double* out, double* lse);

/* Gradients of oracle_sparse_attn for n query rows, given dout [n][Hq][D]
 * (element type `dtype`, 0 or 1 as q, k, v):
 *   dq     : [n][Hq][D]      fp64 out (written)
 *   dk, dv : [*][Hkv][D]     fp64, indexed like k and v, ACCUMULATED into (the
 *                            caller zeroes them)
 * P, the gradient of the logits and everything else is recomputed from q, k,
 * v in fp64; no forward result is taken as input. */
int oracle_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype,
                           const int64_t* kstart, const int64_t* pos, const int32_t* sel,
                           int64_t n, int Hq, int Hkv, int D, int Bk, int topk, double scale,
                           double* dq, double* dk, double* dv);

/* Per-slot block LSE of the main branch for n query rows:
 *   blse : [n][Hq][topk] fp64 out, ln sum over the attended keys of the
 *          slot's block of exp(scale * q . k); -inf for a slot that adds no
 *          block (-1, past the local block, a repeat).  topk <= 32. */
int oracle_block_lse(const void* q, const void* k, int dtype, const int64_t* kstart, const int64_t* pos,
                     const int32_t* sel, int64_t n, int Hq, int Hkv, int D, int Bk, int topk, double scale,
                     double* blse);

/* KL alignment loss of the index branch and its gradients for n query rows
 * (the definition is written out in msa_oracle.c):
 *   loss   : [n][G] fp64 out, KL(A || softmax(S)) per (row, group)
 *   dq_idx : [n][G][DI] fp64 out (written)
 *   dk_idx : [*][DI] fp64, ACCUMULATED into (the caller zeroes it)
 * q_idx / k_idx are read as idx_dtype, q / k (main branch, which defines the
 * target A) as dtype.  G = number of KV heads. */
int oracle_index_kl(const void* q_idx, const void* k_idx, int idx_dtype, const void* q, const void* k,
                    int dtype, const int64_t* kstart, const int64_t* pos, const int32_t* sel, int64_t n, int G,
                    int DI, int Hq, int D, int Bk, int topk, double scale, double* loss, double* dq_idx,
                    double* dk_idx);

/* Index front-end for n tokens (the definition and its readings are written
 * out in msa_oracle.c): hidden states -> projection -> RMS norm -> RoPE.
 *   x      : [n][d_model]        hidden states (dtype)
 *   w_q    : [G*DI][d_model]     index-query projection rows, head g = rows g*DI..
 *   w_k    : [DI][d_model]       index-key projection rows
 *   gain_q, gain_k : [DI]        norm gains
 *   pos    : [n]                 absolute position of each token
 *   q_idx  : [n][G][DI] fp64 out,  k_idx : [n][DI] fp64 out
 * Returns 0, 1 on a bad argument (rope_dim odd or > DI, theta <= 0, eps < 0),
 * 2 when out of memory. */
int oracle_index_frontend(const void* x, const void* w_q, const void* w_k, int dtype, const double* gain_q,
                          const double* gain_k, const int64_t* pos, int64_t n, int d_model, int G, int DI,
                          int rope_dim, double theta, double eps, double* q_idx, double* k_idx);

/* Parameter gradients of the index front-end for upstream gradients dq
 * [n][G][DI] (of q_idx) and dk [n][DI] (of each token's k_idx row), fp64; x is
 * held constant (no dx).  dw_q [G*DI][d_model], dw_k [DI][d_model],
 * dgain_q [DI], dgain_k [DI] are overwritten.  Same return codes. */
int oracle_index_frontend_bwd(const void* x, const void* w_q, const void* w_k, int dtype, const double* gain_q,
                              const double* gain_k, const int64_t* pos, int64_t n, int d_model, int G, int DI,
                              int rope_dim, double theta, double eps, const double* dq, const double* dk,
                              double* dw_q, double* dw_k, double* dgain_q, double* dgain_k);

/* Decode n E4M3 bit patterns to fp32 (exact), for checking the decoder. */
void oracle_decode_e4m3(const uint8_t* in, float* out, int64_t n);

#ifdef __cplusplus
}
#endif
#endif
