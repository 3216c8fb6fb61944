/*
 * CPU oracle for the MSA forward path — TEST INFRASTRUCTURE ONLY (see header).
 *
 * Written from the definitions, one step per function, in double precision:
 *   Eq. 4  block partition           -> block_of()
 *   Eq. 6  index scores + max-pool   -> score_row()
 *   Eq. 7  Top-k, local block forced -> topk_row()
 *   Eq. 8  softmax over the chosen   -> attn_row()
 *   Eq. 9-10 KL alignment per row    -> kl_row()
 *   paged FP8 decode: OCP E4M3 codes -> msa_oracle_fp8_e4m3(), pages looked up
 *   per token
 *   gradients of Eq. 8 (backward)    -> msa_oracle_sparse_attn_bwd(), and the
 *   same gradients on given query rows / one key block -> msa_oracle_sparse_attn_bwd_part()
 * (page "MiniMax Sparse Attention (MSA)" paper review, section 3; page
 * "papers.chlience.com" reading notes, section 5.1 and 5.1.1.)
 * No blocking, fusion or reordering beyond the definitions; OpenMP only
 * splits independent query rows across threads.
 */
#include "msa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16(uint16_t h) {
  uint32_t u = ((uint32_t)h) << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* Eq. 4 (0-based): token j lies in block j / B_k. */
static int64_t block_of(int64_t j, int B_k) { return j / B_k; }

int64_t msa_oracle_num_blocks(int64_t N, int B_k) { return (N + B_k - 1) / B_k; }

int msa_oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Eq. 6 for one query vector qv at position i against keys kidx[0..i]:
 * S_j = <qv, kidx[j]> / sqrt(d_idx), M[b] = max over visible j in block b.
 * Invisible blocks stay -inf (reading notes 5.1.1: invisible tokens are -inf).
 */
static void score_row(const uint16_t* qv, const uint16_t* kidx, int64_t i, int d_idx, int B_k,
                      int64_t B, double* Mrow) {
  double scale = 1.0 / sqrt((double)d_idx);
  for (int64_t b = 0; b < B; ++b) Mrow[b] = -INFINITY;
  for (int64_t j = 0; j <= i; ++j) {
    double s = 0.0;
    for (int d = 0; d < d_idx; ++d) s += bf16(qv[d]) * bf16(kidx[j * d_idx + d]);
    s *= scale;
    int64_t b = block_of(j, B_k);
    if (s > Mrow[b]) Mrow[b] = s;
  }
}

/*
 * Eq. 7 for one (query, group) row.  The local block is always chosen and uses
 * one of the k slots (reading notes 5.1.1); the remaining slots are filled one
 * at a time with the best unchosen earlier block: largest M, and on equal M the
 * lower block index (scan ascending, replace only on strictly greater).
 */
static void topk_row(const double* Mrow, int64_t i, int B_k, int k, int32_t* out, char* chosen) {
  int64_t bl = block_of(i, B_k);
  memset(chosen, 0, (size_t)(bl + 1));
  chosen[bl] = 1;
  int count = 1;
  while (count < k) {
    int64_t best = -1;
    for (int64_t b = 0; b < bl; ++b) {
      if (chosen[b]) continue;
      if (best < 0 || Mrow[b] > Mrow[best]) best = b;
    }
    if (best < 0) break; /* fewer than k causal blocks: all are chosen */
    chosen[best] = 1;
    ++count;
  }
  int n = 0;
  for (int64_t b = 0; b <= bl; ++b)
    if (chosen[b]) out[n++] = (int32_t)b;
  while (n < k) out[n++] = -1;
}

/*
 * Eq. 8 for one head: softmax of scale * <qv, k_j> over the token set
 * T = { j <= i : block_of(j) in the chosen set }, then the weighted sum of v_j.
 * kbase/vbase point at token 0 of this head's group, consecutive tokens are
 * `stride` elements apart.
 */
static void attn_row(const uint16_t* qv, const uint16_t* kbase, const uint16_t* vbase,
                     int64_t stride, int64_t i, int64_t N, int d_h, int B_k, const char* inset,
                     double scale, double* orow, double* lse_out, double* s_buf) {
  int64_t nt = 0;
  double m = -INFINITY;
  int64_t jmax = i < N - 1 ? i : N - 1;
  for (int64_t j = 0; j <= jmax; ++j) {
    if (!inset[block_of(j, B_k)]) continue;
    double s = 0.0;
    for (int d = 0; d < d_h; ++d) s += bf16(qv[d]) * bf16(kbase[j * stride + d]);
    s *= scale;
    s_buf[j] = s;
    if (s > m) m = s;
    ++nt;
  }
  for (int d = 0; d < d_h; ++d) orow[d] = 0.0;
  if (nt == 0) {
    *lse_out = -INFINITY;
    return;
  }
  double l = 0.0;
  for (int64_t j = 0; j <= jmax; ++j) {
    if (!inset[block_of(j, B_k)]) continue;
    double p = exp(s_buf[j] - m);
    l += p;
    for (int d = 0; d < d_h; ++d) orow[d] += p * bf16(vbase[j * stride + d]);
  }
  for (int d = 0; d < d_h; ++d) orow[d] /= l;
  *lse_out = m + log(l);
}

void msa_oracle_block_scores(const uint16_t* q_idx, const uint16_t* k_idx, int64_t N, int H_kv,
                             int d_idx, int B_k, const int64_t* rows, int64_t nrows, double* M) {
  int64_t B = msa_oracle_num_blocks(N, B_k);
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t n = 0; n < nrows; ++n) {
    int64_t i = rows ? rows[n] : n;
    for (int r = 0; r < H_kv; ++r)
      score_row(q_idx + (i * H_kv + r) * d_idx, k_idx, i, d_idx, B_k, B, M + (n * H_kv + r) * B);
  }
}

void msa_oracle_topk(const double* M, const int64_t* rows, int64_t nrows, int H_kv, int64_t B,
                     int B_k, int k, int32_t* block_idx) {
#pragma omp parallel
  {
    char* chosen = (char*)malloc((size_t)B + 1);
#pragma omp for schedule(dynamic, 16)
    for (int64_t n = 0; n < nrows; ++n) {
      int64_t i = rows ? rows[n] : n;
      for (int r = 0; r < H_kv; ++r)
        topk_row(M + (n * H_kv + r) * B, i, B_k, k, block_idx + (n * H_kv + r) * k, chosen);
    }
    free(chosen);
  }
}

void msa_oracle_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const int32_t* block_idx, int64_t N, int H_q, int H_kv, int d_h,
                            int B_k, int kk, double scale, const int64_t* rows, int64_t nrows,
                            double* o, double* lse) {
  int64_t B = msa_oracle_num_blocks(N, B_k);
  int G = H_q / H_kv;
#pragma omp parallel
  {
    char* inset = (char*)malloc((size_t)B);
    double* s_buf = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t n = 0; n < nrows; ++n) {
      int64_t i = rows ? rows[n] : n;
      for (int h = 0; h < H_q; ++h) {
        int r = h / G;
        memset(inset, 0, (size_t)B);
        const int32_t* sel = block_idx + (n * H_kv + r) * kk;
        for (int s = 0; s < kk; ++s)
          if (sel[s] >= 0 && sel[s] < B) inset[sel[s]] = 1;
        attn_row(q + (i * H_q + h) * d_h, k + (int64_t)r * d_h, v + (int64_t)r * d_h,
                 (int64_t)H_kv * d_h, i, N, d_h, B_k, inset, scale, o + (n * H_q + h) * d_h,
                 lse + n * H_q + h, s_buf);
      }
    }
    free(s_buf);
    free(inset);
  }
}

void msa_oracle_decode(const uint16_t* q, const uint16_t* q_idx, const uint16_t* k_cache,
                       const uint16_t* v_cache, const uint16_t* k_idx_cache,
                       const int64_t* cu_seqlens, int batch, int H_q, int H_kv, int d_h,
                       int d_idx, int B_k, int kk, double scale, int32_t* block_idx, double* o,
                       double* lse, double* M, int64_t Bmax) {
  int G = H_q / H_kv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int s = 0; s < batch; ++s) {
    int64_t j0 = cu_seqlens[s];
    int64_t L = cu_seqlens[s + 1] - j0;
    if (L <= 0) continue;
    int64_t i = L - 1; /* the new token is the last cache entry */
    int64_t B = msa_oracle_num_blocks(L, B_k);
    double* Mrow = (double*)malloc(sizeof(double) * (size_t)B);
    char* chosen = (char*)malloc((size_t)B + 1);
    double* s_buf = (double*)malloc(sizeof(double) * (size_t)L);
    for (int r = 0; r < H_kv; ++r) {
      score_row(q_idx + ((int64_t)s * H_kv + r) * d_idx, k_idx_cache + j0 * d_idx, i, d_idx, B_k,
                B, Mrow);
      if (M) {
        double* Mo = M + ((int64_t)s * H_kv + r) * Bmax;
        for (int64_t b = 0; b < Bmax; ++b) Mo[b] = b < B ? Mrow[b] : -INFINITY;
      }
      int32_t* sel = block_idx + ((int64_t)s * H_kv + r) * kk;
      topk_row(Mrow, i, B_k, kk, sel, chosen);
      memset(chosen, 0, (size_t)B);
      for (int t = 0; t < kk; ++t)
        if (sel[t] >= 0) chosen[sel[t]] = 1;
      for (int g = 0; g < G; ++g) {
        int h = r * G + g;
        attn_row(q + ((int64_t)s * H_q + h) * d_h, k_cache + j0 * H_kv * d_h + (int64_t)r * d_h,
                 v_cache + j0 * H_kv * d_h + (int64_t)r * d_h, (int64_t)H_kv * d_h, i, L, d_h,
                 B_k, chosen, scale, o + ((int64_t)s * H_q + h) * d_h, lse + (int64_t)s * H_q + h,
                 s_buf);
      }
    }
    free(s_buf);
    free(chosen);
    free(Mrow);
  }
}

void msa_oracle_decode_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                            const int64_t* cu_seqlens, int batch, int H_q, int H_kv, int d_h,
                            int B_k, int kk, double scale, const int32_t* block_idx_in, double* o,
                            double* lse) {
  int G = H_q / H_kv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int s = 0; s < batch; ++s) {
    int64_t j0 = cu_seqlens[s];
    int64_t L = cu_seqlens[s + 1] - j0;
    if (L <= 0) continue;
    int64_t i = L - 1;
    int64_t B = msa_oracle_num_blocks(L, B_k);
    char* inset = (char*)malloc((size_t)B);
    double* s_buf = (double*)malloc(sizeof(double) * (size_t)L);
    for (int r = 0; r < H_kv; ++r) {
      memset(inset, 0, (size_t)B);
      const int32_t* sel = block_idx_in + ((int64_t)s * H_kv + r) * kk;
      for (int t = 0; t < kk; ++t)
        if (sel[t] >= 0 && sel[t] < B) inset[sel[t]] = 1;
      for (int g = 0; g < G; ++g) {
        int h = r * G + g;
        attn_row(q + ((int64_t)s * H_q + h) * d_h, k_cache + j0 * H_kv * d_h + (int64_t)r * d_h,
                 v_cache + j0 * H_kv * d_h + (int64_t)r * d_h, (int64_t)H_kv * d_h, i, L, d_h, B_k,
                 inset, scale, o + ((int64_t)s * H_q + h) * d_h, lse + (int64_t)s * H_q + h, s_buf);
      }
    }
    free(s_buf);
    free(inset);
  }
}

/*
 * Eq. 9-10 for one (query, group) row.  T is the selected token set (tokens j <= i
 * of the chosen blocks).  The index distribution is the softmax of the index
 * scores over T; the teacher is the mean over the group's G heads of each head's
 * Main Branch softmax over T.  Returns KL(teacher || index) and writes the log
 * partition of the index scores over T.  An empty T gives 0 and -inf.
 */
static double kl_row(const uint16_t* qh0, const uint16_t* kbase, int64_t kstride, const uint16_t* qiv,
                     const uint16_t* kidx, int64_t i, int64_t N, int G, int d_h, int d_idx, int B_k,
                     const char* inset, double scale, double* lse_idx_out, int64_t* tok, double* sidx,
                     double* s_buf, double* P) {
  int64_t nt = 0;
  int64_t jmax = i < N - 1 ? i : N - 1;
  for (int64_t j = 0; j <= jmax; ++j)
    if (inset[block_of(j, B_k)]) tok[nt++] = j;
  if (nt == 0) {
    *lse_idx_out = -INFINITY;
    return 0.0;
  }
  /* index distribution (Eq. 9, left) through its log partition */
  double mi = -INFINITY;
  for (int64_t t = 0; t < nt; ++t) {
    double sv = 0.0;
    for (int d = 0; d < d_idx; ++d) sv += bf16(qiv[d]) * bf16(kidx[tok[t] * d_idx + d]);
    sidx[t] = sv / sqrt((double)d_idx);
    if (sidx[t] > mi) mi = sidx[t];
  }
  double li = 0.0;
  for (int64_t t = 0; t < nt; ++t) li += exp(sidx[t] - mi);
  double lse_idx = mi + log(li);
  *lse_idx_out = lse_idx;
  /* teacher (Eq. 9, right): mean over heads of each head's softmax over T */
  for (int64_t t = 0; t < nt; ++t) P[t] = 0.0;
  for (int g = 0; g < G; ++g) {
    const uint16_t* qv = qh0 + (int64_t)g * d_h;
    double m = -INFINITY;
    for (int64_t t = 0; t < nt; ++t) {
      double sv = 0.0;
      for (int d = 0; d < d_h; ++d) sv += bf16(qv[d]) * bf16(kbase[tok[t] * kstride + d]);
      s_buf[t] = sv * scale;
      if (s_buf[t] > m) m = s_buf[t];
    }
    double l = 0.0;
    for (int64_t t = 0; t < nt; ++t) l += exp(s_buf[t] - m);
    for (int64_t t = 0; t < nt; ++t) P[t] += exp(s_buf[t] - m) / l / G;
  }
  /* Eq. 10 summand: KL(P || P_idx) = sum_j P_j (log P_j - log P_idx_j) */
  double kl = 0.0;
  for (int64_t t = 0; t < nt; ++t)
    if (P[t] > 0.0) kl += P[t] * (log(P[t]) - (sidx[t] - lse_idx));
  return kl;
}

void msa_oracle_sparse_kl(const uint16_t* q, const uint16_t* k, const uint16_t* q_idx,
                          const uint16_t* k_idx, const int32_t* block_idx, int64_t N, int H_q,
                          int H_kv, int d_h, int d_idx, int B_k, int kk, double scale,
                          const int64_t* rows, int64_t nrows, double* kl, double* lse_idx) {
  int64_t B = msa_oracle_num_blocks(N, B_k);
  int G = H_q / H_kv;
#pragma omp parallel
  {
    size_t cap = (size_t)(N > 0 ? N : 1);
    char* inset = (char*)malloc((size_t)B + 1);
    int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * cap);
    double* sidx = (double*)malloc(sizeof(double) * cap);
    double* s_buf = (double*)malloc(sizeof(double) * cap);
    double* P = (double*)malloc(sizeof(double) * cap);
#pragma omp for schedule(dynamic, 1)
    for (int64_t n = 0; n < nrows; ++n) {
      int64_t i = rows ? rows[n] : n;
      for (int r = 0; r < H_kv; ++r) {
        memset(inset, 0, (size_t)B + 1);
        const int32_t* sel = block_idx + (n * H_kv + r) * kk;
        for (int s = 0; s < kk; ++s)
          if (sel[s] >= 0 && sel[s] < B) inset[sel[s]] = 1;
        kl[n * H_kv + r] = kl_row(q + (i * H_q + (int64_t)r * G) * d_h, k + (int64_t)r * d_h,
                                  (int64_t)H_kv * d_h, q_idx + (i * H_kv + r) * d_idx, k_idx, i, N, G,
                                  d_h, d_idx, B_k, inset, scale, lse_idx + n * H_kv + r, tok, sidx,
                                  s_buf, P);
      }
    }
    free(P);
    free(s_buf);
    free(sidx);
    free(tok);
    free(inset);
  }
}

/*
 * OCP FP8 E4M3 (the "fn" variant: no infinities, S.1111.111 is NaN): 1 sign bit,
 * 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
 * subnormals m/8 * 2^-6.
 */
double msa_oracle_fp8_e4m3(uint8_t x) {
  int sgn = x >> 7, e = (x >> 3) & 15, m = x & 7;
  double v;
  if (e == 15 && m == 7) return NAN;
  if (e == 0)
    v = ldexp(m / 8.0, -6);
  else
    v = ldexp(1.0 + m / 8.0, e - 7);
  return sgn ? -v : v;
}

void msa_oracle_decode_paged(const uint16_t* q, const uint16_t* q_idx, const uint8_t* k_pages,
                             const uint8_t* v_pages, double k_scale, double v_scale,
                             const uint16_t* kidx_pages, const int32_t* block_table,
                             int64_t max_blocks, const int64_t* seqlens, int batch, int H_q,
                             int H_kv, int d_h, int d_idx, int B_k, int kk, double scale,
                             const int32_t* block_idx_in, int32_t* block_idx, double* o, double* lse,
                             double* M, int64_t Bmax) {
  int G = H_q / H_kv;
#pragma omp parallel for schedule(dynamic, 1)
  for (int s = 0; s < batch; ++s) {
    int64_t L = seqlens[s];
    if (L <= 0) continue;
    int64_t i = L - 1; /* the new token is the last cached token */
    int64_t B = msa_oracle_num_blocks(L, B_k);
    const int32_t* pages = block_table + (int64_t)s * max_blocks;
    /* the sequence's index keys in token order, gathered from its pages */
    uint16_t* kidx = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)L * d_idx);
    for (int64_t j = 0; j < L; ++j)
      memcpy(kidx + j * d_idx, kidx_pages + ((int64_t)pages[j / B_k] * B_k + j % B_k) * d_idx,
             sizeof(uint16_t) * d_idx);
    double* Mrow = (double*)malloc(sizeof(double) * (size_t)B);
    char* chosen = (char*)malloc((size_t)B + 1);
    double* s_buf = (double*)malloc(sizeof(double) * (size_t)L);
    for (int r = 0; r < H_kv; ++r) {
      score_row(q_idx + ((int64_t)s * H_kv + r) * d_idx, kidx, i, d_idx, B_k, B, Mrow);
      if (M) {
        double* Mo = M + ((int64_t)s * H_kv + r) * Bmax;
        for (int64_t b = 0; b < Bmax; ++b) Mo[b] = b < B ? Mrow[b] : -INFINITY;
      }
      int32_t* sel = block_idx + ((int64_t)s * H_kv + r) * kk;
      if (block_idx_in) /* attention on a given selection */
        memcpy(sel, block_idx_in + ((int64_t)s * H_kv + r) * kk, sizeof(int32_t) * kk);
      else
        topk_row(Mrow, i, B_k, kk, sel, chosen);
      memset(chosen, 0, (size_t)B);
      for (int t = 0; t < kk; ++t)
        if (sel[t] >= 0 && sel[t] < B) chosen[sel[t]] = 1;
      /* Eq. 8 with K = k_scale * code, V = v_scale * code, read through the pages */
      for (int g = 0; g < G; ++g) {
        int h = r * G + g;
        const uint16_t* qv = q + ((int64_t)s * H_q + h) * d_h;
        double m = -INFINITY;
        for (int64_t j = 0; j <= i; ++j) {
          if (!chosen[block_of(j, B_k)]) continue;
          const uint8_t* kr = k_pages + (((int64_t)pages[j / B_k] * B_k + j % B_k) * H_kv + r) * d_h;
          double sv = 0.0;
          for (int d = 0; d < d_h; ++d) sv += bf16(qv[d]) * (k_scale * msa_oracle_fp8_e4m3(kr[d]));
          s_buf[j] = sv * scale;
          if (s_buf[j] > m) m = s_buf[j];
        }
        double* orow = o + ((int64_t)s * H_q + h) * d_h;
        for (int d = 0; d < d_h; ++d) orow[d] = 0.0;
        double l = 0.0;
        for (int64_t j = 0; j <= i; ++j) {
          if (!chosen[block_of(j, B_k)]) continue;
          const uint8_t* vr = v_pages + (((int64_t)pages[j / B_k] * B_k + j % B_k) * H_kv + r) * d_h;
          double p = exp(s_buf[j] - m);
          l += p;
          for (int d = 0; d < d_h; ++d) orow[d] += p * (v_scale * msa_oracle_fp8_e4m3(vr[d]));
        }
        for (int d = 0; d < d_h; ++d) orow[d] /= l;
        lse[(int64_t)s * H_q + h] = m + log(l);
      }
    }
    free(s_buf);
    free(chosen);
    free(Mrow);
    free(kidx);
  }
}

/*
 * Gradients of Eq. 8 with respect to q, k and v for the upstream gradient dO of o
 * (the selection is held fixed).  Per query i and head h of group r, over the token
 * set T of reading 6: P_j = softmax_j(scale <q, k_j>), o = sum_j P_j v_j, and with
 * D = <dO, o>:  dv_j += P_j dO,  dS_j = P_j (<dO, v_j> - D),
 * dq += scale sum_j dS_j k_j,  dk_j += scale dS_j q.
 * Threads split the KV groups, so the key/value gradients of a group have one writer.
 */
void msa_oracle_sparse_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const uint16_t* dO, const int32_t* block_idx, int64_t N, int H_q,
                                int H_kv, int d_h, int B_k, int kk, double scale, double* dq,
                                double* dk, double* dv) {
  int64_t B = msa_oracle_num_blocks(N, B_k);
  int G = H_q / H_kv;
  for (int64_t e = 0; e < N * H_q * d_h; ++e) dq[e] = 0.0;
  for (int64_t e = 0; e < N * H_kv * d_h; ++e) dk[e] = dv[e] = 0.0;
#pragma omp parallel for schedule(dynamic, 1)
  for (int r = 0; r < H_kv; ++r) {
    char* inset = (char*)malloc((size_t)B + 1);
    double* P = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double* o = (double*)malloc(sizeof(double) * (size_t)d_h);
    for (int64_t i = 0; i < N; ++i) {
      memset(inset, 0, (size_t)B + 1);
      const int32_t* sel = block_idx + (i * H_kv + r) * kk;
      for (int t = 0; t < kk; ++t)
        if (sel[t] >= 0 && sel[t] < B) inset[sel[t]] = 1;
      for (int g = 0; g < G; ++g) {
        int h = r * G + g;
        const uint16_t* qv = q + (i * H_q + h) * d_h;
        const uint16_t* dov = dO + (i * H_q + h) * d_h;
        /* forward: softmax over T and o */
        double m = -INFINITY;
        int64_t nt = 0;
        for (int64_t j = 0; j <= i; ++j) {
          if (!inset[block_of(j, B_k)]) continue;
          const uint16_t* kr = k + (j * H_kv + r) * d_h;
          double sv = 0.0;
          for (int d = 0; d < d_h; ++d) sv += bf16(qv[d]) * bf16(kr[d]);
          P[j] = sv * scale;
          if (P[j] > m) m = P[j];
          ++nt;
        }
        if (nt == 0) continue; /* no token: o = 0, no gradient */
        double l = 0.0;
        for (int64_t j = 0; j <= i; ++j)
          if (inset[block_of(j, B_k)]) {
            P[j] = exp(P[j] - m);
            l += P[j];
          }
        for (int d = 0; d < d_h; ++d) o[d] = 0.0;
        for (int64_t j = 0; j <= i; ++j) {
          if (!inset[block_of(j, B_k)]) continue;
          P[j] /= l;
          const uint16_t* vr = v + (j * H_kv + r) * d_h;
          for (int d = 0; d < d_h; ++d) o[d] += P[j] * bf16(vr[d]);
        }
        double D = 0.0;
        for (int d = 0; d < d_h; ++d) D += bf16(dov[d]) * o[d];
        /* backward */
        double* dqr = dq + (i * H_q + h) * d_h;
        for (int64_t j = 0; j <= i; ++j) {
          if (!inset[block_of(j, B_k)]) continue;
          const uint16_t* kr = k + (j * H_kv + r) * d_h;
          const uint16_t* vr = v + (j * H_kv + r) * d_h;
          double dp = 0.0;
          for (int d = 0; d < d_h; ++d) dp += bf16(dov[d]) * bf16(vr[d]);
          double ds = P[j] * (dp - D);
          double* dkr = dk + (j * H_kv + r) * d_h;
          double* dvr = dv + (j * H_kv + r) * d_h;
          for (int d = 0; d < d_h; ++d) {
            dqr[d] += scale * ds * bf16(kr[d]);
            dkr[d] += scale * ds * bf16(qv[d]);
            dvr[d] += P[j] * bf16(dov[d]);
          }
        }
      }
    }
    free(o);
    free(P);
    free(inset);
  }
}

/*
 * One (query i, head h of group r) row of the backward of Eq. 8: the softmax P over
 * the row's token set T (tokens j <= i of the blocks marked in inset), o and
 * D = <dO, o>, then dS_j = P_j (<dO, V_j> - D).  When dqr is given it receives
 * scale * sum_j dS_j K_j; tokens j in [jlo, jhi) add scale * dS_j * q to dk and
 * P_j * dO to dv (rows j - jlo).  P is scratch of at least i + 1 doubles.
 * Returns 0 when T is empty (no gradient).
 */
static int bwd_row(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dO,
                   const char* inset, int64_t i, int r, int h, int H_q, int H_kv, int d_h, int B_k,
                   double scale, double* P, double* o, double* dqr, int64_t jlo, int64_t jhi,
                   double* dk, double* dv) {
  const uint16_t* qv = q + (i * H_q + h) * d_h;
  const uint16_t* dov = dO + (i * H_q + h) * d_h;
  double m = -INFINITY;
  int64_t nt = 0;
  for (int64_t j = 0; j <= i; ++j) {
    if (!inset[block_of(j, B_k)]) continue;
    const uint16_t* kr = k + (j * H_kv + r) * d_h;
    double sv = 0.0;
    for (int d = 0; d < d_h; ++d) sv += bf16(qv[d]) * bf16(kr[d]);
    P[j] = sv * scale;
    if (P[j] > m) m = P[j];
    ++nt;
  }
  if (nt == 0) return 0;
  double l = 0.0;
  for (int64_t j = 0; j <= i; ++j)
    if (inset[block_of(j, B_k)]) {
      P[j] = exp(P[j] - m);
      l += P[j];
    }
  for (int d = 0; d < d_h; ++d) o[d] = 0.0;
  for (int64_t j = 0; j <= i; ++j) {
    if (!inset[block_of(j, B_k)]) continue;
    P[j] /= l;
    const uint16_t* vr = v + (j * H_kv + r) * d_h;
    for (int d = 0; d < d_h; ++d) o[d] += P[j] * bf16(vr[d]);
  }
  double D = 0.0;
  for (int d = 0; d < d_h; ++d) D += bf16(dov[d]) * o[d];
  for (int64_t j = 0; j <= i; ++j) {
    if (!inset[block_of(j, B_k)]) continue;
    const int in_blk = j >= jlo && j < jhi;
    if (!dqr && !in_blk) continue;
    const uint16_t* kr = k + (j * H_kv + r) * d_h;
    const uint16_t* vr = v + (j * H_kv + r) * d_h;
    double dp = 0.0;
    for (int d = 0; d < d_h; ++d) dp += bf16(dov[d]) * bf16(vr[d]);
    double ds = P[j] * (dp - D);
    if (dqr)
      for (int d = 0; d < d_h; ++d) dqr[d] += scale * ds * bf16(kr[d]);
    if (in_blk) {
      double* dkr = dk + (j - jlo) * d_h;
      double* dvr = dv + (j - jlo) * d_h;
      for (int d = 0; d < d_h; ++d) {
        dkr[d] += scale * ds * bf16(qv[d]);
        dvr[d] += P[j] * bf16(dov[d]);
      }
    }
  }
  return 1;
}

/* Marks the blocks of one (query, group) selection row in inset (B + 1 entries). */
static void mark_row(const int32_t* sel, int kk, int64_t B, char* inset) {
  memset(inset, 0, (size_t)B + 1);
  for (int t = 0; t < kk; ++t)
    if (sel[t] >= 0 && sel[t] < B) inset[sel[t]] = 1;
}

void msa_oracle_sparse_attn_bwd_part(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const uint16_t* dO, const int32_t* block_idx, int64_t N, int H_q,
                                     int H_kv, int d_h, int B_k, int kk, double scale, const int64_t* rows,
                                     int64_t nrows, double* dq_rows, int64_t kb, int kr, double* dk_blk,
                                     double* dv_blk) {
  int64_t B = msa_oracle_num_blocks(N, B_k);
  int G = H_q / H_kv;
  for (int64_t e = 0; e < nrows * H_q * d_h; ++e) dq_rows[e] = 0.0;
  /* dq of the listed rows: each row's own softmax and its selected tokens. */
#pragma omp parallel
  {
    char* inset = (char*)malloc((size_t)B + 1);
    double* P = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double* o = (double*)malloc(sizeof(double) * (size_t)d_h);
#pragma omp for schedule(dynamic, 1)
    for (int64_t a = 0; a < nrows; ++a) {
      int64_t i = rows[a];
      for (int r = 0; r < H_kv; ++r) {
        mark_row(block_idx + (i * H_kv + r) * kk, kk, B, inset);
        for (int g = 0; g < G; ++g)
          bwd_row(q, k, v, dO, inset, i, r, r * G + g, H_q, H_kv, d_h, B_k, scale, P, o,
                  dq_rows + (a * H_q + r * G + g) * d_h, 0, 0, NULL, NULL);
      }
    }
    free(o);
    free(P);
    free(inset);
  }
  if (kb < 0 || kb >= B || kr < 0 || kr >= H_kv) return;
  /* dk, dv of key block kb of group kr: every query row whose selection holds kb. */
  int64_t jlo = kb * B_k, jhi = (kb + 1) * B_k < N ? (kb + 1) * B_k : N;
  int64_t nb = (int64_t)B_k * d_h;
  for (int64_t e = 0; e < nb; ++e) dk_blk[e] = dv_blk[e] = 0.0;
  int nth = msa_oracle_threads();
  double* acc = (double*)calloc((size_t)nth * 2 * (size_t)nb, sizeof(double));
#pragma omp parallel num_threads(nth)
  {
    int t = 0;
#ifdef _OPENMP
    t = omp_get_thread_num();
#endif
    double* dk_t = acc + (size_t)t * 2 * nb;
    double* dv_t = dk_t + nb;
    char* inset = (char*)malloc((size_t)B + 1);
    double* P = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double* o = (double*)malloc(sizeof(double) * (size_t)d_h);
#pragma omp for schedule(static)
    for (int64_t i = jlo; i < N; ++i) {
      mark_row(block_idx + (i * H_kv + kr) * kk, kk, B, inset);
      if (!inset[kb]) continue;
      for (int g = 0; g < G; ++g)
        bwd_row(q, k, v, dO, inset, i, kr, kr * G + g, H_q, H_kv, d_h, B_k, scale, P, o, NULL, jlo, jhi,
                dk_t, dv_t);
    }
    free(o);
    free(P);
    free(inset);
  }
  for (int t = 0; t < nth; ++t)
    for (int64_t e = 0; e < nb; ++e) {
      dk_blk[e] += acc[(size_t)t * 2 * nb + e];
      dv_blk[e] += acc[(size_t)t * 2 * nb + nb + e];
    }
  free(acc);
}
