/*
 * CPU oracle for the MSA (MiniMax Sparse Attention) forward path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library links, includes or calls
 * this code; only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no source with the GPU path.
 *
 * Plain loops in double precision over the same bf16 input bytes the GPU sees.
 * Each function follows one step of the pages (page "MiniMax Sparse Attention
 * (MSA)" paper review, section 3 "core formulas", Eq. 4, 6, 7, 8, 9, 10; page
 * "papers.chlience.com" reading notes, section 5.1.1 "block Top-k procedure").
 *
 * Conventions shared by all functions:
 *   - bf16 tensors are passed as uint16_t bit patterns, row-major, contiguous.
 *   - "rows" lists the query positions to evaluate (nrows of them); rows == NULL
 *     means every position 0..N-1 (then nrows must equal N).
 *   - Blocks are 0-based: block b covers tokens [b*B_k, min((b+1)*B_k, N)).
 */
#ifndef MSA_ORACLE_H
#define MSA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Eq. 4: number of blocks B = ceil(N / B_k). */
int64_t msa_oracle_num_blocks(int64_t N, int B_k);

/* Threads OpenMP will use (reported with CPU timings). */
int msa_oracle_threads(void);

/*
 * Eq. 6: M[n][r][b] = max over j in block b with j <= i of
 *        <q_idx[i][r], k_idx[j]> / sqrt(d_idx),  i = rows[n].
 * Blocks with no visible token (b > i / B_k) are -inf.
 * q_idx: [N][H_kv][d_idx], k_idx: [N][d_idx], M: [nrows][H_kv][B] (double).
 */
void msa_oracle_block_scores(const uint16_t* q_idx, const uint16_t* k_idx, int64_t N, int H_kv,
                             int d_idx, int B_k, const int64_t* rows, int64_t nrows, double* M);

/*
 * Eq. 7 with the forced local block: for row n (position i = rows[n]) and group r,
 * the local block b_loc = i / B_k takes one of the k slots; the other k-1 slots go
 * to the highest M among blocks b < b_loc, ties to the lower block index.  If
 * b_loc + 1 <= k every causal block is chosen.  Output ascending, padded with -1.
 * M: [nrows][H_kv][B], block_idx: [nrows][H_kv][k].
 */
void msa_oracle_topk(const double* M, const int64_t* rows, int64_t nrows, int H_kv, int64_t B,
                     int B_k, int k, int32_t* block_idx);

/*
 * Eq. 8 (with causality from Eq. 1-2): for row n (position i), head h of group
 * r = h / (H_q / H_kv), softmax over the tokens j <= i whose block is listed in
 * block_idx[n][r][:] (entries < 0 or >= B are ignored; the list is a set).
 *   o[n][h][:] = sum_j p_j v[j][r][:],  lse[n][h] = log sum_j exp(s_j),
 *   s_j = scale * <q[i][h], k[j][r]>.
 * An empty token set gives o = 0 and lse = -inf.
 * q: [N][H_q][d_h]; k, v: [N][H_kv][d_h]; block_idx: [nrows][H_kv][kk];
 * o: [nrows][H_q][d_h]; lse: [nrows][H_q] (double).
 */
void msa_oracle_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const int32_t* block_idx, int64_t N, int H_q, int H_kv, int d_h,
                            int B_k, int kk, double scale, const int64_t* rows, int64_t nrows,
                            double* o, double* lse);

/*
 * Decode: one new token per sequence, already stored as the last cache entry
 * (position L_s - 1 of sequence s).  Steps as above on that one query.
 * q: [batch][H_q][d_h]; q_idx: [batch][H_kv][d_idx];
 * k_cache, v_cache: [T][H_kv][d_h]; k_idx_cache: [T][d_idx]; cu_seqlens: [batch+1];
 * outputs block_idx: [batch][H_kv][kk], o: [batch][H_q][d_h], lse: [batch][H_q];
 * M (optional, may be NULL): [batch][H_kv][Bmax] with Bmax = ceil(max L / B_k).
 */
void msa_oracle_decode(const uint16_t* q, const uint16_t* q_idx, const uint16_t* k_cache,
                       const uint16_t* v_cache, const uint16_t* k_idx_cache,
                       const int64_t* cu_seqlens, int batch, int H_q, int H_kv, int d_h,
                       int d_idx, int B_k, int kk, double scale, int32_t* block_idx, double* o,
                       double* lse, double* M, int64_t Bmax);

/*
 * Decode attention only (Eq. 8 for the last token of each sequence) on a given
 * selection block_idx_in [batch][H_kv][kk] (entries < 0 ignored; a set).
 */
void msa_oracle_decode_attn(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                            const int64_t* cu_seqlens, int batch, int H_q, int H_kv, int d_h,
                            int B_k, int kk, double scale, const int32_t* block_idx_in, double* o,
                            double* lse);

/*
 * Eq. 9-10 (KL alignment) for row n (position i) and group r, over the selected
 * token set T = { j <= i : block_of(j) listed in block_idx[n][r][:] }:
 *   P_idx(j) = softmax over T of S_idx(j) = <q_idx[i][r], k_idx[j]> / sqrt(d_idx),
 *   P(j)     = (1/G) sum over the group's heads h of softmax over T of
 *              scale * <q[i][h], k[j][r]>,
 *   kl[n][r] = sum over j in T of P(j) log(P(j) / P_idx(j))  (0 log 0 = 0),
 *   lse_idx[n][r] = log sum over j in T of exp(S_idx(j)).
 * Empty T: kl = 0, lse_idx = -inf.  The loss of Eq. 10 is the mean of kl over all
 * (i, r).  kl, lse_idx: [nrows][H_kv] (double).
 */
void msa_oracle_sparse_kl(const uint16_t* q, const uint16_t* k, const uint16_t* q_idx,
                          const uint16_t* k_idx, const int32_t* block_idx, int64_t N, int H_q,
                          int H_kv, int d_h, int d_idx, int B_k, int kk, double scale,
                          const int64_t* rows, int64_t nrows, double* kl, double* lse_idx);

/* OCP FP8 E4M3 ("fn": no infinities, S.1111.111 is NaN) code -> value. */
double msa_oracle_fp8_e4m3(uint8_t x);

/*
 * Decode over a paged cache: pages of B_k tokens; token j of sequence s is row
 * j % B_k of page block_table[s][j / B_k] (block_table: [batch][max_blocks]).
 * k_pages, v_pages: [P][B_k][H_kv][d_h] FP8 E4M3 codes with K = k_scale * value,
 * V = v_scale * value; kidx_pages: [P][B_k][d_idx] bf16; seqlens: [batch].  The new
 * token is the last cached one (position L_s - 1).  Outputs as msa_oracle_decode;
 * with block_idx_in (not NULL) that selection is used (and copied to block_idx)
 * instead of the Top-k.
 */
void msa_oracle_decode_paged(const uint16_t* q, const uint16_t* q_idx, const uint8_t* k_pages,
                             const uint8_t* v_pages, double k_scale, double v_scale,
                             const uint16_t* kidx_pages, const int32_t* block_table,
                             int64_t max_blocks, const int64_t* seqlens, int batch, int H_q,
                             int H_kv, int d_h, int d_idx, int B_k, int kk, double scale,
                             const int32_t* block_idx_in, int32_t* block_idx, double* o, double* lse,
                             double* M, int64_t Bmax);

/*
 * Gradients of Eq. 8 (selection fixed) for the upstream gradient dO [N][H_q][d_h]
 * (bf16): dq [N][H_q][d_h], dk, dv [N][H_kv][d_h] (double), all rows of the
 * block_idx [N][H_kv][kk] given.  Rows with no attended token get no gradient.
 */
void msa_oracle_sparse_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                const uint16_t* dO, const int32_t* block_idx, int64_t N, int H_q,
                                int H_kv, int d_h, int B_k, int kk, double scale, double* dq,
                                double* dk, double* dv);

/*
 * The same gradients restricted, for checks at sizes where the full backward is too
 * slow: dq_rows [nrows][H_q][d_h] for the listed query rows, and dk_blk, dv_blk
 * [B_k][d_h] for the tokens of key block kb of group kr (every query row whose
 * selection holds kb contributes; rows of the block past N stay 0).  kb < 0 skips
 * the block part.
 */
void msa_oracle_sparse_attn_bwd_part(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const uint16_t* dO, const int32_t* block_idx, int64_t N, int H_q,
                                     int H_kv, int d_h, int B_k, int kk, double scale, const int64_t* rows,
                                     int64_t nrows, double* dq_rows, int64_t kb, int kr, double* dk_blk,
                                     double* dv_blk);

#ifdef __cplusplus
}
#endif
#endif
