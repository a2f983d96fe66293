/*
 * msa_oracle.c -- plain CPU oracle for MiniMax Sparse Attention (MSA).
 *
 * TEST INFRASTRUCTURE ONLY: called by the tests, by the smoke check and by the
 * CPU-baseline leg of the benchmark, never by the product path.  It shares no
 * code with the GPU library.  Every step is written out exactly as the method
 * defines it, with no blocking, fusion or reordering; the only parallelism is
 * an OpenMP loop over independent query rows.
 *
 * Sources (page title, section):
 *   [P4] "MiniMax Sparse Attention: let each query pick its own blocks",
 *        section "The mechanism, precisely" (index branch / main branch) and
 *        the paper's Figure 1 caption reproduced there.
 *   [P5] atlas record of MiniMax M3 (atlas.lewiswon.me), summary paragraph
 *        ("max-pooled dot products", top-k = 16 of 128-token blocks, local
 *        block forced, standard scaled dot-product softmax attention).
 *   [P1] "llama.cpp Merges MiniMax M3's Sparse Attention ...", key facts:
 *        16 blocks of 128 tokens, always including the block being written.
 *
 * Readings taken where the pages are silent are listed in msa_oracle.h.
 */
#include "msa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* E4M3: value = (-1)^s * (1 + m/8) * 2^(e-7) for e > 0, (-1)^s * (m/8) * 2^-6
 * for e = 0; e = 15 with m = 7 is NaN (there is no infinity). */
static float e4m3_to_float(uint8_t v) {
  const int s = v >> 7, e = (v >> 3) & 15, m = v & 7;
  float x;
  if (e == 15 && m == 7) x = NAN;
  else if (e == 0) x = ldexpf((float)m, -9);
  else x = ldexpf((float)(8 + m), e - 10);
  return s ? -x : x;
}

void oracle_decode_e4m3(const uint8_t* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = e4m3_to_float(in[i]);
}

static float load_elem(const void* base, int dtype, int64_t i) {
  if (dtype == 0) return ((const float*)base)[i];
  if (dtype == 2) return e4m3_to_float(((const uint8_t*)base)[i]);
  uint32_t bits = ((uint32_t)((const uint16_t*)base)[i]) << 16; /* bf16 -> fp32, exact */
  float f;
  memcpy(&f, &bits, sizeof f);
  return f;
}

static int64_t floor_div(int64_t a, int64_t b) {
  int64_t q = a / b;
  if ((a % b != 0) && ((a < 0) != (b < 0))) q -= 1;
  return q;
}

typedef struct {
  float score;
  int32_t block;
} scored_block;

/* Total order of the selection: higher pooled score first; equal scores are
 * broken towards the lower block id (the deterministic tie-break). */
static int by_score_then_block(const void* pa, const void* pb) {
  const scored_block* a = (const scored_block*)pa;
  const scored_block* b = (const scored_block*)pb;
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
  return (a->block > b->block) - (a->block < b->block);
}

static int ascending_int(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

/* [P4] index branch: token score s_j = q_idx . k_idx[j] (raw dot product,
 * no scale: selection is "exp-free", on raw scores [P5]); block score
 * S_c = max of s_j over the Bk tokens of block c [P4 Figure 1 "block max
 * pooling"]; keep the local block l = floor(p / Bk) and the best k-1 earlier
 * blocks c < l [P4, P5]. */
int oracle_index_topk(const void* q_idx, const void* k_idx, int dtype,
                      const int64_t* kstart, const int64_t* pos, int64_t n,
                      int G, int DI, int Bk, int topk, int32_t* sel,
                      float* scores, int64_t nbmax) {
  if (!q_idx || !k_idx || !kstart || !pos || !sel) return 1;
  if (n < 0 || G <= 0 || DI <= 0 || Bk <= 0 || topk <= 0) return 1;
  if (dtype != 0 && dtype != 1 && dtype != 2) return 1;

  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t r = 0; r < n; ++r) {
    const int64_t p = pos[r];
    const int64_t local = floor_div(p, Bk);
    const int64_t nearlier = local > 0 ? local : 0; /* blocks c < local */
    if (scores && nearlier > nbmax) { bad = 1; continue; }
    scored_block* cand = (scored_block*)malloc(sizeof(scored_block) * (size_t)(nearlier > 0 ? nearlier : 1));
    int32_t* chosen = (int32_t*)malloc(sizeof(int32_t) * (size_t)topk);
    if (!cand || !chosen) { bad = 1; free(cand); free(chosen); continue; }

    for (int g = 0; g < G; ++g) {
      int32_t* out = sel + (r * G + g) * (int64_t)topk;
      for (int i = 0; i < topk; ++i) out[i] = -1;
      if (scores)
        for (int64_t c = 0; c < nbmax; ++c) scores[(r * G + g) * nbmax + c] = -INFINITY;
      if (p < 0) continue; /* no key is visible */

      const int64_t qoff = (r * G + g) * (int64_t)DI;
      for (int64_t c = 0; c < nearlier; ++c) {
        float best = -INFINITY;
        for (int64_t j = c * Bk; j < (c + 1) * Bk; ++j) {
          const int64_t koff = (kstart[r] + j) * (int64_t)DI;
          float s = 0.0f; /* fp32, sequential over d */
          for (int d = 0; d < DI; ++d)
            s += load_elem(q_idx, dtype, qoff + d) * load_elem(k_idx, dtype, koff + d);
          if (s > best) best = s;
        }
        cand[c].score = best;
        cand[c].block = (int32_t)c;
        if (scores) scores[(r * G + g) * nbmax + c] = best;
      }

      qsort(cand, (size_t)nearlier, sizeof(scored_block), by_score_then_block);
      int64_t keep = nearlier < (int64_t)(topk - 1) ? nearlier : (int64_t)(topk - 1);
      int cnt = 0;
      for (int64_t i = 0; i < keep; ++i) chosen[cnt++] = cand[i].block;
      chosen[cnt++] = (int32_t)local; /* the local block is always kept */
      qsort(chosen, (size_t)cnt, sizeof(int32_t), ascending_int);
      for (int i = 0; i < cnt; ++i) out[i] = chosen[i];
    }
    free(cand);
    free(chosen);
  }
  return bad;
}

/* [P4] main branch: exact softmax attention over the keys of the selected
 * blocks, for every head of the group, with the causal limit j <= p inside
 * the local block.  z_j = scale * q . k_j; o = sum_j softmax(z)_j v_j;
 * lse = log sum_j exp(z_j).  All in fp64. */
int oracle_sparse_attn_kv(const void* q, const void* k, const void* v, int dtype, int kv_dtype,
                          const int64_t* kstart, const int64_t* pos, const int32_t* sel,
                          int64_t n, int Hq, int Hkv, int D, int Bk, int topk,
                          double scale, double* out, double* lse) {
  if (!q || !k || !v || !kstart || !pos || !sel || !out || !lse) return 1;
  if (n < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Bk <= 0 || topk <= 0) return 1;
  if (Hq % Hkv != 0) return 1;
  if (dtype != 0 && dtype != 1 && dtype != 2) return 1;
  if (kv_dtype != 0 && kv_dtype != 1 && kv_dtype != 2) return 1;
  const int r_heads = Hq / Hkv;

  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t r = 0; r < n; ++r) {
    int32_t* blocks = (int32_t*)malloc(sizeof(int32_t) * (size_t)topk);
    double* z = (double*)malloc(sizeof(double) * (size_t)topk * (size_t)Bk);
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)topk * (size_t)Bk);
    if (!blocks || !z || !keys) { bad = 1; free(blocks); free(z); free(keys); continue; }
    const int64_t p = pos[r];

    for (int h = 0; h < Hq; ++h) {
      const int g = h / r_heads; /* contiguous GQA grouping */
      double* o = out + (r * Hq + h) * (int64_t)D;
      for (int d = 0; d < D; ++d) o[d] = 0.0;

      /* J = { j <= p : floor(j / Bk) in Sel }, Sel taken as a set. */
      int nb = 0;
      for (int i = 0; i < topk; ++i) {
        int32_t c = sel[(r * Hkv + g) * (int64_t)topk + i];
        if (c >= 0) blocks[nb++] = c;
      }
      qsort(blocks, (size_t)nb, sizeof(int32_t), ascending_int);
      int64_t nk = 0;
      for (int i = 0; i < nb; ++i) {
        if (i > 0 && blocks[i] == blocks[i - 1]) continue;
        for (int64_t j = (int64_t)blocks[i] * Bk; j < ((int64_t)blocks[i] + 1) * Bk; ++j)
          if (j <= p) keys[nk++] = j;
      }
      if (nk == 0) { lse[r * Hq + h] = -INFINITY; continue; }

      const int64_t qoff = (r * Hq + h) * (int64_t)D;
      double m = -INFINITY;
      for (int64_t a = 0; a < nk; ++a) {
        const int64_t koff = ((kstart[r] + keys[a]) * Hkv + g) * (int64_t)D;
        double dot = 0.0;
        for (int d = 0; d < D; ++d)
          dot += (double)load_elem(q, dtype, qoff + d) * (double)load_elem(k, kv_dtype, koff + d);
        z[a] = scale * dot;
        if (z[a] > m) m = z[a];
      }
      double l = 0.0;
      for (int64_t a = 0; a < nk; ++a) {
        const double w = exp(z[a] - m);
        l += w;
        const int64_t voff = ((kstart[r] + keys[a]) * Hkv + g) * (int64_t)D;
        for (int d = 0; d < D; ++d) o[d] += w * (double)load_elem(v, kv_dtype, voff + d);
      }
      for (int d = 0; d < D; ++d) o[d] /= l;
      lse[r * Hq + h] = m + log(l);
    }
    free(blocks);
    free(z);
    free(keys);
  }
  return bad;
}

int oracle_sparse_attn(const void* q, const void* k, const void* v, int dtype,
                       const int64_t* kstart, const int64_t* pos, const int32_t* sel,
                       int64_t n, int Hq, int Hkv, int D, int Bk, int topk,
                       double scale, double* out, double* lse) {
  return oracle_sparse_attn_kv(q, k, v, dtype, dtype, kstart, pos, sel, n, Hq, Hkv, D, Bk, topk, scale,
                               out, lse);
}

/* Gradients of the main branch ([P4] "The mechanism, precisely": the main
 * branch is ordinary softmax attention over the selected keys, so its
 * gradients are those of softmax attention restricted to J).  For one row and
 * head, with P_j = exp(z_j) / sum_i exp(z_i) over j in J and dO the gradient
 * of the output:
 *   dP_j  = dO . v_j
 *   delta = sum_j P_j dP_j
 *   dS_j  = P_j (dP_j - delta)          (gradient of the logit z_j)
 *   dq   += scale * sum_j dS_j k_j
 *   dk_j += scale * dS_j q               (summed over rows and the group's heads)
 *   dv_j += P_j dO
 * All in fp64.  dq is written; dk and dv are accumulated (the caller zeroes
 * them); rows run in parallel, each thread summing its rows' dk / dv
 * contributions into a private buffer that is added at the end. */
int oracle_sparse_attn_bwd(const void* q, const void* k, const void* v, const void* dout, int dtype,
                           const int64_t* kstart, const int64_t* pos, const int32_t* sel,
                           int64_t n, int Hq, int Hkv, int D, int Bk, int topk, double scale,
                           double* dq, double* dk, double* dv) {
  if (!q || !k || !v || !dout || !kstart || !pos || !sel || !dq || !dk || !dv) return 1;
  if (n < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Bk <= 0 || topk <= 0) return 1;
  if (Hq % Hkv != 0) return 1;
  if (dtype != 0 && dtype != 1) return 1;
  const int r_heads = Hq / Hkv;

  /* dk and dv cover every key row any query row reaches */
  int64_t nkeys = 0;
  for (int64_t r = 0; r < n; ++r)
    if (pos[r] >= 0 && kstart[r] + pos[r] + 1 > nkeys) nkeys = kstart[r] + pos[r] + 1;
  const size_t kv_elems = (size_t)nkeys * (size_t)Hkv * (size_t)D;

  int bad = 0;
#pragma omp parallel reduction(| : bad)
  {
    /* each thread sums its rows' dk / dv contributions privately; the
     * per-thread sums are added at the end */
    double* my_dk = (double*)calloc(kv_elems ? kv_elems : 1, sizeof(double));
    double* my_dv = (double*)calloc(kv_elems ? kv_elems : 1, sizeof(double));
    int32_t* blocks = (int32_t*)malloc(sizeof(int32_t) * (size_t)topk);
    double* z = (double*)malloc(sizeof(double) * (size_t)topk * (size_t)Bk);
    double* dp = (double*)malloc(sizeof(double) * (size_t)topk * (size_t)Bk);
    int64_t* keys = (int64_t*)malloc(sizeof(int64_t) * (size_t)topk * (size_t)Bk);
    const int ok = my_dk && my_dv && blocks && z && dp && keys;
    if (!ok) bad = 1;
#pragma omp for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
      if (!ok) continue;
      const int64_t p = pos[r];
      for (int h = 0; h < Hq; ++h) {
        const int g = h / r_heads;
        double* dqh = dq + (r * Hq + h) * (int64_t)D;
        for (int d = 0; d < D; ++d) dqh[d] = 0.0;

        /* J as in the forward definition: Sel taken as a set, keys j <= p */
        int nb = 0;
        for (int i = 0; i < topk; ++i) {
          int32_t c = sel[(r * Hkv + g) * (int64_t)topk + i];
          if (c >= 0) blocks[nb++] = c;
        }
        qsort(blocks, (size_t)nb, sizeof(int32_t), ascending_int);
        int64_t nk = 0;
        for (int i = 0; i < nb; ++i) {
          if (i > 0 && blocks[i] == blocks[i - 1]) continue;
          for (int64_t j = (int64_t)blocks[i] * Bk; j < ((int64_t)blocks[i] + 1) * Bk; ++j)
            if (j <= p) keys[nk++] = j;
        }
        if (nk == 0) continue;

        const int64_t qoff = (r * Hq + h) * (int64_t)D;
        double m = -INFINITY;
        for (int64_t a = 0; a < nk; ++a) {
          const int64_t koff = ((kstart[r] + keys[a]) * Hkv + g) * (int64_t)D;
          double dot = 0.0;
          for (int d = 0; d < D; ++d)
            dot += (double)load_elem(q, dtype, qoff + d) * (double)load_elem(k, dtype, koff + d);
          z[a] = scale * dot;
          if (z[a] > m) m = z[a];
        }
        double l = 0.0;
        for (int64_t a = 0; a < nk; ++a) {
          z[a] = exp(z[a] - m);
          l += z[a];
        }
        double delta = 0.0;
        for (int64_t a = 0; a < nk; ++a) {
          z[a] /= l; /* z now holds P */
          const int64_t voff = ((kstart[r] + keys[a]) * Hkv + g) * (int64_t)D;
          double dot = 0.0;
          for (int d = 0; d < D; ++d)
            dot += (double)load_elem(dout, dtype, qoff + d) * (double)load_elem(v, dtype, voff + d);
          dp[a] = dot;
          delta += z[a] * dot;
        }
        for (int64_t a = 0; a < nk; ++a) {
          const double ds = z[a] * (dp[a] - delta);
          const int64_t koff = ((kstart[r] + keys[a]) * Hkv + g) * (int64_t)D;
          for (int d = 0; d < D; ++d) {
            dqh[d] += scale * ds * (double)load_elem(k, dtype, koff + d);
            my_dk[koff + d] += scale * ds * (double)load_elem(q, dtype, qoff + d);
            my_dv[koff + d] += z[a] * (double)load_elem(dout, dtype, qoff + d);
          }
        }
      }
    }
#pragma omp critical
    {
      if (ok)
        for (size_t i = 0; i < kv_elems; ++i) {
          dk[i] += my_dk[i];
          dv[i] += my_dv[i];
        }
    }
    free(my_dk);
    free(my_dv);
    free(blocks);
    free(z);
    free(dp);
    free(keys);
  }
  return bad;
}

/* The distinct attended blocks of one selection row (Sel taken as a set):
 * slot i is attended when its id is >= 0, at or before the local block and
 * not a repeat of an earlier slot.  Returns a bit mask of those slots. */
static unsigned valid_slots(const int32_t* row_sel, int topk, int64_t local) {
  unsigned mask = 0;
  for (int i = 0; i < topk; ++i) {
    const int32_t c = row_sel[i];
    int ok = c >= 0 && c <= local;
    for (int j = 0; j < i && ok; ++j) ok = row_sel[j] != c;
    if (ok) mask |= 1u << i;
  }
  return mask;
}

/* Per-slot block LSE of the main branch: for row r, head h and selection slot
 * i naming block c, ln sum over the attended keys j of block c (j <= p) of
 * exp(z_j), z_j = scale * q . k_j in fp64; -inf for a slot that adds no
 * block.  exp(blse - lse) is the share of the head's attention in the block. */
int oracle_block_lse(const void* q, const void* k, int dtype, const int64_t* kstart, const int64_t* pos,
                     const int32_t* sel, int64_t n, int Hq, int Hkv, int D, int Bk, int topk, double scale,
                     double* blse) {
  if (!q || !k || !kstart || !pos || !sel || !blse) return 1;
  if (n < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Bk <= 0 || topk <= 0 || topk > 32) return 1;
  if (Hq % Hkv != 0) return 1;
  if (dtype != 0 && dtype != 1 && dtype != 2) return 1;
  const int r_heads = Hq / Hkv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t r = 0; r < n; ++r) {
    const int64_t p = pos[r];
    for (int h = 0; h < Hq; ++h) {
      const int g = h / r_heads;
      const int32_t* rs = sel + (r * Hkv + g) * (int64_t)topk;
      const unsigned mask = p >= 0 ? valid_slots(rs, topk, floor_div(p, Bk)) : 0u;
      const int64_t qoff = (r * Hq + h) * (int64_t)D;
      for (int i = 0; i < topk; ++i) {
        double* out = blse + (r * Hq + h) * (int64_t)topk + i;
        if (!((mask >> i) & 1u)) { *out = -INFINITY; continue; }
        const int64_t j0 = (int64_t)rs[i] * Bk;
        const int64_t j1 = j0 + Bk - 1 < p ? j0 + Bk - 1 : p;
        double m = -INFINITY;
        for (int64_t j = j0; j <= j1; ++j) {
          const int64_t koff = ((kstart[r] + j) * Hkv + g) * (int64_t)D;
          double dot = 0.0;
          for (int d = 0; d < D; ++d)
            dot += (double)load_elem(q, dtype, qoff + d) * (double)load_elem(k, dtype, koff + d);
          if (scale * dot > m) m = scale * dot;
        }
        double l = 0.0;
        for (int64_t j = j0; j <= j1; ++j) {
          const int64_t koff = ((kstart[r] + j) * Hkv + g) * (int64_t)D;
          double dot = 0.0;
          for (int d = 0; d < D; ++d)
            dot += (double)load_elem(q, dtype, qoff + d) * (double)load_elem(k, dtype, koff + d);
          l += exp(scale * dot - m);
        }
        *out = m + log(l);
      }
    }
  }
  return 0;
}

/* KL alignment of the index branch ([P4] "Two design choices": an auxiliary
 * KL loss aligns the index branch's block scores with the main attention's
 * distribution over blocks; [P5] summary: against the group-averaged main
 * distribution, with a stop-gradient so only the index projections learn).
 * For row r and group g, over the attended slots i of its selection:
 *   A_i = (1/r_heads) sum_{h in g} exp(blse[h][i] - lse[h])  main branch's
 *         share of attention in block c_i, averaged over the group's heads
 *         (blse, lse: oracle_block_lse and the logsumexp over the slots)
 *   S_i = max over the attended keys j of block c_i of q_idx . k_idx[j]
 *         (fp32, sequential over d, as the index branch scores; the lowest j
 *         among equal maxima is the argmax j*_i)
 *   I   = softmax over the attended slots of S (fp64)
 *   loss[r][g] = sum_i A_i (ln A_i - ln I_i)   (terms with A_i = 0 are 0)
 * A is a constant target (no gradient reaches q, k); the gradients of the
 * sum of loss[r][g] over all rows and groups with respect to S are
 *   dS_i = I_i (sum_k A_k) - A_i,
 * and through the max: dq_idx[r][g] = sum_i dS_i k_idx[j*_i] (written),
 * dk_idx[j*_i] += dS_i q_idx[r][g] (accumulated; the caller zeroes it). */
int oracle_index_kl(const void* q_idx, const void* k_idx, int idx_dtype, const void* q, const void* k,
                    int dtype, const int64_t* kstart, const int64_t* pos, const int32_t* sel, int64_t n, int G,
                    int DI, int Hq, int D, int Bk, int topk, double scale, double* loss, double* dq_idx,
                    double* dk_idx) {
  if (!q_idx || !k_idx || !q || !k || !kstart || !pos || !sel || !loss || !dq_idx || !dk_idx) return 1;
  if (n < 0 || G <= 0 || DI <= 0 || Hq <= 0 || D <= 0 || Bk <= 0 || topk <= 0 || topk > 32) return 1;
  if (Hq % G != 0) return 1;
  if (idx_dtype != 0 && idx_dtype != 1 && idx_dtype != 2) return 1;
  const int r_heads = Hq / G;
  double* blse = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1) * (size_t)Hq * (size_t)topk);
  if (!blse) return 1;
  if (oracle_block_lse(q, k, dtype, kstart, pos, sel, n, Hq, G, D, Bk, topk, scale, blse) != 0) {
    free(blse);
    return 1;
  }
  int64_t nkeys = 0;
  for (int64_t r = 0; r < n; ++r)
    if (pos[r] >= 0 && kstart[r] + pos[r] + 1 > nkeys) nkeys = kstart[r] + pos[r] + 1;
  const size_t kv_elems = (size_t)nkeys * (size_t)DI;

  int bad = 0;
#pragma omp parallel reduction(| : bad)
  {
    double* my_dk = (double*)calloc(kv_elems ? kv_elems : 1, sizeof(double));
    if (!my_dk) bad = 1;
#pragma omp for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
      if (!my_dk) continue;
      const int64_t p = pos[r];
      for (int g = 0; g < G; ++g) {
        double* dq = dq_idx + (r * G + g) * (int64_t)DI;
        for (int d = 0; d < DI; ++d) dq[d] = 0.0;
        loss[r * G + g] = 0.0;
        const int32_t* rs = sel + (r * G + g) * (int64_t)topk;
        const unsigned mask = p >= 0 ? valid_slots(rs, topk, floor_div(p, Bk)) : 0u;
        if (!mask) continue;
        double A[32], S[32], I[32];
        int64_t jstar[32];
        const int64_t qoff = (r * G + g) * (int64_t)DI;
        for (int i = 0; i < topk; ++i) {
          if (!((mask >> i) & 1u)) continue;
          /* main branch share of block i, averaged over the group's heads */
          double a = 0.0;
          for (int hh = 0; hh < r_heads; ++hh) {
            const int h = g * r_heads + hh;
            const double* bl = blse + (r * Hq + h) * (int64_t)topk;
            double m = -INFINITY, l = 0.0;
            for (int k2 = 0; k2 < topk; ++k2)
              if (bl[k2] > m) m = bl[k2];
            for (int k2 = 0; k2 < topk; ++k2)
              if (bl[k2] > -INFINITY) l += exp(bl[k2] - m);
            a += exp(bl[i] - (m + log(l)));
          }
          A[i] = a / r_heads;
          /* index score and argmax over the block's attended keys */
          const int64_t j0 = (int64_t)rs[i] * Bk;
          const int64_t j1 = j0 + Bk - 1 < p ? j0 + Bk - 1 : p;
          float best = -INFINITY;
          int64_t bj = j0;
          for (int64_t j = j0; j <= j1; ++j) {
            float s = 0.0f;
            const int64_t koff = (kstart[r] + j) * (int64_t)DI;
            for (int d = 0; d < DI; ++d)
              s += load_elem(q_idx, idx_dtype, qoff + d) * load_elem(k_idx, idx_dtype, koff + d);
            if (s > best) { best = s; bj = j; }
          }
          S[i] = (double)best;
          jstar[i] = bj;
        }
        double m = -INFINITY, z = 0.0, asum = 0.0;
        for (int i = 0; i < topk; ++i)
          if ((mask >> i) & 1u && S[i] > m) m = S[i];
        for (int i = 0; i < topk; ++i)
          if ((mask >> i) & 1u) z += exp(S[i] - m);
        double ls = 0.0;
        for (int i = 0; i < topk; ++i) {
          if (!((mask >> i) & 1u)) continue;
          I[i] = exp(S[i] - m) / z;
          asum += A[i];
          if (A[i] > 0.0) ls += A[i] * (log(A[i]) - (S[i] - m - log(z)));
        }
        loss[r * G + g] = ls;
        for (int i = 0; i < topk; ++i) {
          if (!((mask >> i) & 1u)) continue;
          const double ds = I[i] * asum - A[i];
          const int64_t koff = (kstart[r] + jstar[i]) * (int64_t)DI;
          for (int d = 0; d < DI; ++d) {
            dq[d] += ds * (double)load_elem(k_idx, idx_dtype, koff + d);
            my_dk[koff + d] += ds * (double)load_elem(q_idx, idx_dtype, qoff + d);
          }
        }
      }
    }
#pragma omp critical
    {
      if (my_dk)
        for (size_t i = 0; i < kv_elems; ++i) dk_idx[i] += my_dk[i];
    }
    free(my_dk);
  }
  free(blse);
  return bad;
}

/* Index front-end: [P4] Figure 1 caption (the index branch takes the hidden
 * states through a linear projection, a norm and RoPE to its index-query
 * heads, one per GQA group, and its single shared index-key head, [P5]
 * summary paragraph).  The pages give the order of the three steps, the model
 * width (3072) and, for the main heads, a rotary width of half the 128-dim
 * head ([P5] provenance, section 5.1); the norm's kind and the rotary base are
 * not given.  Readings, for every head vector separately:
 *   projection : y = W_h x, W_h the DI rows of head h, no bias;
 *   norm       : y_i <- gain_i * y_i / sqrt(mean_i(y_i^2) + eps) over the DI
 *                values (one gain vector for the query heads, one for the key
 *                head);
 *   RoPE       : for i < rope_dim/2 the pair (y_i, y_{i+rope_dim/2}) is turned
 *                by the angle p * theta^(-2i/rope_dim), p the token's absolute
 *                position: (a, b) -> (a cos - b sin, b cos + a sin); values at
 *                i >= rope_dim pass through.
 * Everything in fp64 after an exact widening of x and W. */
int oracle_index_frontend(const void* x, const void* w_q, const void* w_k, int dtype, const double* gain_q,
                          const double* gain_k, const int64_t* pos, int64_t n, int d_model, int G, int DI,
                          int rope_dim, double theta, double eps, double* q_idx, double* k_idx) {
  if (n < 0 || d_model <= 0 || G <= 0 || DI <= 0 || rope_dim < 0 || rope_dim > DI || (rope_dim & 1) ||
      !(theta > 0.0) || !(eps >= 0.0))
    return 1;
  /* widen the G+1 heads' weight rows once: row h*DI + i of wd is row i of head h */
  const int64_t wrows = (int64_t)(G + 1) * DI;
  double* wd = malloc((size_t)wrows * d_model * sizeof(double));
  if (!wd) return 2;
  for (int64_t rw = 0; rw < wrows; ++rw) {
    const void* w = rw < (int64_t)G * DI ? w_q : w_k;
    const int64_t src = rw < (int64_t)G * DI ? rw : rw - (int64_t)G * DI;
    for (int c = 0; c < d_model; ++c) wd[rw * d_model + c] = (double)load_elem(w, dtype, src * d_model + c);
  }
  const int half = rope_dim / 2;
  int bad = 0;
#pragma omp parallel
  {
    double* xr = malloc((size_t)d_model * sizeof(double));
    double* y = malloc((size_t)DI * sizeof(double));
    if (!xr || !y) {
#pragma omp atomic write
      bad = 2;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < n; ++r) {
      if (!xr || !y) continue;
      for (int c = 0; c < d_model; ++c) xr[c] = (double)load_elem(x, dtype, r * d_model + c);
      for (int h = 0; h <= G; ++h) {
        for (int i = 0; i < DI; ++i) {
          const double* wrow = wd + ((int64_t)h * DI + i) * d_model;
          double s = 0.0;
          for (int c = 0; c < d_model; ++c) s += wrow[c] * xr[c];
          y[i] = s;
        }
        double ms = 0.0;
        for (int i = 0; i < DI; ++i) ms += y[i] * y[i];
        const double inv = 1.0 / sqrt(ms / DI + eps);
        const double* gain = h < G ? gain_q : gain_k;
        for (int i = 0; i < DI; ++i) y[i] = gain[i] * (y[i] * inv);
        for (int i = 0; i < half; ++i) {
          const double ang = (double)pos[r] * pow(theta, -2.0 * i / rope_dim);
          const double cs = cos(ang), sn = sin(ang);
          const double a = y[i], b = y[i + half];
          y[i] = a * cs - b * sn;
          y[i + half] = b * cs + a * sn;
        }
        double* out = h < G ? q_idx + (r * G + h) * DI : k_idx + r * DI;
        memcpy(out, y, (size_t)DI * sizeof(double));
      }
    }
    free(xr);
    free(y);
  }
  free(wd);
  return bad;
}

/* Gradients of the index front-end with respect to its parameters, for
 * upstream gradients dq (of q_idx) and dk (of k_idx).  The indexer's input x
 * is held constant ([P5] summary: the alignment loss reaches only the index
 * projections, through a stop-gradient on the indexer's input), so there is
 * no dx.  Per head vector, with n = y / r, r = sqrt(mean(y^2) + eps),
 * z = gain * n and out = R z (R the rotation written out above):
 *   dz      = R^T dout                       (each pair turned back by -angle)
 *   dgain  += dz * n
 *   dn      = dz * gain
 *   dy      = (dn - n * (dn . n) / DI) / r
 *   dW_h   += dy x^T
 * All in fp64.  dw_q [G*DI][d_model], dw_k [DI][d_model], dgain_q [DI],
 * dgain_k [DI] are overwritten. */
int oracle_index_frontend_bwd(const void* x, const void* w_q, const void* w_k, int dtype, const double* gain_q,
                              const double* gain_k, const int64_t* pos, int64_t n, int d_model, int G, int DI,
                              int rope_dim, double theta, double eps, const double* dq, const double* dk,
                              double* dw_q, double* dw_k, double* dgain_q, double* dgain_k) {
  if (n < 0 || d_model <= 0 || G <= 0 || DI <= 0 || rope_dim < 0 || rope_dim > DI || (rope_dim & 1) ||
      !(theta > 0.0) || !(eps >= 0.0))
    return 1;
  const int64_t wrows = (int64_t)(G + 1) * DI;
  const size_t wsize = (size_t)wrows * d_model;
  double* wd = malloc(wsize * sizeof(double));
  if (!wd) return 2;
  for (int64_t rw = 0; rw < wrows; ++rw) {
    const void* w = rw < (int64_t)G * DI ? w_q : w_k;
    const int64_t src = rw < (int64_t)G * DI ? rw : rw - (int64_t)G * DI;
    for (int c = 0; c < d_model; ++c) wd[rw * d_model + c] = (double)load_elem(w, dtype, src * d_model + c);
  }
  memset(dw_q, 0, (size_t)G * DI * d_model * sizeof(double));
  memset(dw_k, 0, (size_t)DI * d_model * sizeof(double));
  memset(dgain_q, 0, (size_t)DI * sizeof(double));
  memset(dgain_k, 0, (size_t)DI * sizeof(double));
  const int half = rope_dim / 2;
  int bad = 0;
#pragma omp parallel
  {
    double* xr = malloc((size_t)d_model * sizeof(double));
    double* y = malloc((size_t)DI * sizeof(double));
    double* dz = malloc((size_t)DI * sizeof(double));
    double* my_dw = calloc(wsize, sizeof(double));
    double* my_dg = calloc(2 * (size_t)DI, sizeof(double));
    if (!xr || !y || !dz || !my_dw || !my_dg) {
#pragma omp atomic write
      bad = 2;
    }
#pragma omp for schedule(dynamic, 4)
    for (int64_t r = 0; r < n; ++r) {
      if (!xr || !y || !dz || !my_dw || !my_dg) continue;
      for (int c = 0; c < d_model; ++c) xr[c] = (double)load_elem(x, dtype, r * d_model + c);
      for (int h = 0; h <= G; ++h) {
        for (int i = 0; i < DI; ++i) {
          const double* wrow = wd + ((int64_t)h * DI + i) * d_model;
          double s = 0.0;
          for (int c = 0; c < d_model; ++c) s += wrow[c] * xr[c];
          y[i] = s;
        }
        double ms = 0.0;
        for (int i = 0; i < DI; ++i) ms += y[i] * y[i];
        const double rr = sqrt(ms / DI + eps);
        const double* dout = h < G ? dq + (r * G + h) * DI : dk + r * DI;
        for (int i = 0; i < DI; ++i) dz[i] = dout[i];
        for (int i = 0; i < half; ++i) {
          const double ang = (double)pos[r] * pow(theta, -2.0 * i / rope_dim);
          const double cs = cos(ang), sn = sin(ang);
          const double a = dz[i], b = dz[i + half];
          dz[i] = a * cs + b * sn;
          dz[i + half] = b * cs - a * sn;
        }
        const double* gain = h < G ? gain_q : gain_k;
        double* dg = my_dg + (h < G ? 0 : DI);
        double dot = 0.0;
        for (int i = 0; i < DI; ++i) {
          const double nv = y[i] / rr;
          dg[i] += dz[i] * nv;
          dot += dz[i] * gain[i] * nv;
        }
        double* dwh = my_dw + (int64_t)h * DI * d_model;
        for (int i = 0; i < DI; ++i) {
          const double nv = y[i] / rr;
          const double dy = (dz[i] * gain[i] - nv * dot / DI) / rr;
          double* row = dwh + (int64_t)i * d_model;
          for (int c = 0; c < d_model; ++c) row[c] += dy * xr[c];
        }
      }
    }
#pragma omp critical
    {
      if (my_dw && my_dg) {
        for (size_t i = 0; i < (size_t)G * DI * d_model; ++i) dw_q[i] += my_dw[i];
        for (size_t i = 0; i < (size_t)DI * d_model; ++i) dw_k[i] += my_dw[(size_t)G * DI * d_model + i];
        for (int i = 0; i < DI; ++i) {
          dgain_q[i] += my_dg[i];
          dgain_k[i] += my_dg[DI + i];
        }
      }
    }
    free(xr);
    free(y);
    free(dz);
    free(my_dw);
    free(my_dg);
  }
  free(wd);
  return bad;
}
