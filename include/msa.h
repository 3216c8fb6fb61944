/*
 * msa.h — C ABI of the MSA (MiniMax Sparse Attention) forward path on AMD
 * Instinct MI355X (gfx950).
 *
 * The method (page "MiniMax Sparse Attention (MSA)" paper review, section 3):
 *   Index Branch  — Eq. 6: every causal token j <= i is scored per GQA group r
 *                   with one index-query head against one shared index-key
 *                   head, S = <Q_idx[i,r], K_idx[j]> / sqrt(d_idx); the scores
 *                   are max-pooled per block of B_k keys (Eq. 4 partition);
 *                 — Eq. 7: the k best blocks are kept per (query, group) without
 *                   any exponential; the query's own (local) block is always
 *                   kept and uses one of the k slots (reading notes page,
 *                   section 5.1.1).
 *   Main Branch   — Eq. 8: exact softmax attention of every head of group r over
 *                   the tokens of the kept blocks, causal inside the local block.
 *
 * Conventions for every call
 *   - All tensors live in device memory, row-major and contiguous, and must be
 *     16-byte aligned.  bf16 tensors are passed as raw device pointers.
 *   - The caller owns every buffer, including the workspace whose size the
 *     matching *_workspace() query returns.  The library keeps no device memory
 *     between calls, holds no state and is re-entrant per stream.
 *   - Calls are asynchronous on `hip_stream` (a hipStream_t passed as void*;
 *     NULL = the default stream) and never synchronise.
 *   - Arguments are checked on the host before anything is launched; a bad call
 *     returns a status and writes nothing.  No call aborts or throws.  A failed
 *     launch returns MSA_ERR_HIP.  msa_last_error() describes the last failure
 *     on the calling thread.
 *   - Blocks are numbered from 0: block b holds tokens [b*B_k, min((b+1)*B_k, N)).
 *     Head h belongs to group h / (H_q / H_kv) (adjacent heads share a KV head).
 *   - Supported shapes: d_h = 128, d_idx = 64, B_k = 64 or 128, 1 <= k <= 32,
 *     H_q / H_kv a power of two <= 128 and ceil(N / B_k) <= 8192 (N <= 2^20 at
 *     B_k = 128, 2^19 at 64).
 *     Other shapes return MSA_ERR_UNSUPPORTED.  N = 0 (or batch = 0) is a valid
 *     empty call that launches nothing.
 *   - Same inputs give bitwise-identical outputs (no atomics touch results).
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = 1, /* null/misaligned pointer, negative size, inconsistent shape */
  MSA_ERR_UNSUPPORTED = 2, /* shape outside the supported set above */
  MSA_ERR_WORKSPACE = 3,   /* workspace pointer null or smaller than required */
  MSA_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} msa_status_t;

const char* msa_status_string(msa_status_t status);
const char* msa_last_error(void);

/* ------------------------------------------------------------------ Index Branch
 * msa_index_topk — Eq. 6 + Eq. 7 with the forced local block.
 *   q_idx     bf16 [N, H_kv, d_idx]   index queries (one head per group)
 *   k_idx     bf16 [N, d_idx]         shared index keys
 *   block_idx int32 [N, H_kv, k]      out: per (query, group) the chosen blocks,
 *             ascending, padded with -1 when fewer than k blocks are causal
 *             (b_loc + 1 < k).  Ties in block score go to the lower block index.
 * The N x N token scores and the block scores are never written to memory.
 * Needs no workspace (msa_index_topk_workspace returns 0; ws may be NULL).
 */
size_t msa_index_topk_workspace(int64_t N, int H_kv, int d_idx, int B_k, int k);
msa_status_t msa_index_topk(const void* q_idx, const void* k_idx, int64_t N, int H_kv, int d_idx,
                            int B_k, int k, int32_t* block_idx, void* ws, size_t ws_bytes,
                            void* hip_stream);

/* ------------------------------------------------------------------ Main Branch
 * msa_sparse_attn_fwd — Eq. 8 over the blocks listed in block_idx.
 *   q         bf16 [N, H_q, d_h];  k, v  bf16 [N, H_kv, d_h]
 *   block_idx int32 [N, H_kv, k]  entries < 0 or >= ceil(N/B_k) are ignored;
 *             entries past the query's local block add no token (causal);
 *             each block may appear at most once per row (repeats are counted
 *             once per occurrence).
 *   scale     softmax scale applied to <q, k> (the pages use 1/sqrt(d_h))
 *   o         fp32 [N, H_q, d_h]   out: normalised attention output
 *   lse       fp32 [N, H_q]        out: natural-log sum of exp(scale * <q,k>)
 *             over the attended tokens; a row with no token gets o = 0,
 *             lse = -inf.
 * Work runs KV-block-outer (pages: "KV-outer sparse attention" with query
 * gather and a two-phase LSE combine), in query windows whose size follows
 * from ws_bytes: the workspace query returns the size for the default window;
 * any ws_bytes >= msa_sparse_attn_fwd_workspace_min() works (smaller windows).
 */
size_t msa_sparse_attn_fwd_workspace(int64_t N, int H_q, int H_kv, int d_h, int B_k, int k);
size_t msa_sparse_attn_fwd_workspace_min(int64_t N, int H_q, int H_kv, int d_h, int B_k, int k);
/* The number of query windows msa_sparse_attn_fwd runs for this shape with a
 * workspace of ws_bytes (1 when the workspace covers all N queries at once); 0 for
 * N == 0; -1 for an unsupported shape or ws_bytes below the minimum.  Host-only. */
int64_t msa_sparse_attn_fwd_windows(int64_t N, int H_q, int H_kv, int d_h, int B_k, int k, size_t ws_bytes);
msa_status_t msa_sparse_attn_fwd(const void* q, const void* k, const void* v,
                                 const int32_t* block_idx, int64_t N, int H_q, int H_kv, int d_h,
                                 int B_k, int k_sel, float scale, float* o, float* lse, void* ws,
                                 size_t ws_bytes, void* hip_stream);

/* msa_sparse_attn_fwd_lse_idx — msa_sparse_attn_fwd that also emits LSE_idx, the log
 * partition of the index distribution over each row's selected tokens (Eq. 9's
 * P^idx; the paper review page, section 5, 4.3, has the main pass emit such LSE
 * scalars so that the KL term's backward needs no separate forward):
 *   lse_idx[i][r] = ln sum_{j <= i, j in the row's selected blocks} exp(S_j),
 *   S_j = <q_idx[i][r], k_idx[j]> / sqrt(d_idx),
 * -inf for a row with no selected token.  Computed over the forward's own lists
 * (each index-key block staged once per list), after its combine.
 *   q_idx  bf16 [N, H_kv, d_idx];  k_idx  bf16 [N, d_idx];  d_idx = 64
 *   lse_idx fp32 [N, H_kv]  out
 * Everything else (arguments, outputs, workspace sizes, windows, errors) as
 * msa_sparse_attn_fwd; o and lse are bit-identical to its results. */
msa_status_t msa_sparse_attn_fwd_lse_idx(const void* q, const void* k, const void* v,
                                         const void* q_idx, const void* k_idx,
                                         const int32_t* block_idx, int64_t N, int H_q, int H_kv,
                                         int d_h, int d_idx, int B_k, int k_sel, float scale,
                                         float* o, float* lse, float* lse_idx, void* ws,
                                         size_t ws_bytes, void* hip_stream);

/* ------------------------------------------------------------------ KL alignment
 * msa_sparse_kl_fwd — Eq. 9-10 (the Index Branch's alignment loss, Algorithm 1
 * step 7) on the selected token set T of each (query, group): the tokens j <= i
 * of the blocks in block_idx (same rules as msa_sparse_attn_fwd).
 *   P_idx(j) = softmax over T of the index scores <q_idx[i][r], k_idx[j]> / sqrt(d_idx)
 *   P(j)     = mean over the group's G heads of each head's Main Branch softmax
 *              over T, the teacher (scores scale * <q[i][h], k[j][r]>)
 *   kl[i][r] = KL(P || P_idx);  loss = mean of kl over all (i, r)  (Eq. 10)
 * Inputs as for msa_index_topk / msa_sparse_attn_fwd, plus
 *   lse       fp32 [N, H_q]  the log partitions that msa_sparse_attn_fwd emitted
 *             for the same q, k, block_idx and scale (the pages' kernel emits
 *             these scalars in the main pass; the teacher is normalised by them).
 * Outputs (device):
 *   kl        fp32 [N, H_kv]
 *   lse_idx   fp32 [N, H_kv]  log sum over T of exp(index score): the scalar a
 *             backward pass would load; an empty T gives kl = 0, lse_idx = -inf.
 *   loss      fp32 [1]        mean of kl (fixed-order fp64 sum; deterministic).
 * Limits: G = H_q / H_kv <= 32, d_idx = 64, and the other limits of
 * msa_sparse_attn_fwd.  Workspace sizes as for msa_sparse_attn_fwd (its own
 * queries; smaller workspaces run in query windows).
 */
size_t msa_sparse_kl_fwd_workspace(int64_t N, int H_q, int H_kv, int d_h, int d_idx, int B_k,
                                   int k);
size_t msa_sparse_kl_fwd_workspace_min(int64_t N, int H_q, int H_kv, int d_h, int d_idx, int B_k,
                                       int k);
msa_status_t msa_sparse_kl_fwd(const void* q, const void* k, const void* q_idx, const void* k_idx,
                               const int32_t* block_idx, const float* lse, int64_t N, int H_q,
                               int H_kv, int d_h, int d_idx, int B_k, int k_sel, float scale,
                               float* kl, float* lse_idx, float* loss, void* ws, size_t ws_bytes,
                               void* hip_stream);

/* msa_sparse_kl_fwd_from_lse_idx — msa_sparse_kl_fwd with LSE_idx given rather than
 * computed: the forward emits it (msa_sparse_attn_fwd_lse_idx), as the pages' main
 * pass emits its LSE scalars (paper review page, section 5, 4.3), so the KL value
 * needs only the teacher terms: kl = sum_j P(j) (ln P(j) - S_j) + LSE_idx, summed
 * over T (with sum_j P(j) kept exact).
 *   lse_idx  fp32 [N, H_kv] in: LSE_idx for the same q_idx, k_idx and block_idx
 *            (-inf marks an empty T: kl = 0 there)
 * Other arguments, outputs (kl, loss), workspace sizes, limits and errors as
 * msa_sparse_kl_fwd. */
msa_status_t msa_sparse_kl_fwd_from_lse_idx(const void* q, const void* k, const void* q_idx,
                                            const void* k_idx, const int32_t* block_idx,
                                            const float* lse, const float* lse_idx, int64_t N,
                                            int H_q, int H_kv, int d_h, int d_idx, int B_k,
                                            int k_sel, float scale, float* kl, float* loss,
                                            void* ws, size_t ws_bytes, void* hip_stream);

/* ------------------------------------------------------------------ Backward
 * msa_sparse_attn_bwd — gradients of Eq. 8 with respect to q, k and v for the
 * upstream gradient dO of o, the selection block_idx held fixed (reading notes,
 * section 5.4: the backward over data-dependent sparsity).  With P the softmax
 * over each row's selected tokens and D = <dO, o> per (query, head):
 *   dV = P^T dO,  dS = P (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q.
 *   q, k, v, block_idx, scale  as given to msa_sparse_attn_fwd
 *   o, lse     fp32 [N, H_q, d_h], [N, H_q]  that call's outputs
 *   dO         bf16 [N, H_q, d_h]
 *   dq         fp32 [N, H_q, d_h]   out
 *   dk, dv     fp32 [N, H_kv, d_h]  out (overwritten, not accumulated into)
 * Limits: G = H_q / H_kv <= 32, and those of msa_sparse_attn_fwd (B_k = 64 or 128).
 * Workspace as for the forward (smaller workspaces run in query windows), with a
 * default size capped at 64 GiB rather than 40 GiB (one window at 128K).  No
 * atomics touch a gradient and each block's rows are listed in (query, slot) order,
 * so all three gradients are bitwise reproducible across reruns with the same
 * workspace size; dq also across workspace sizes, while dk and dv then group their
 * per-window sums differently (fp32 rounding level).
 */
size_t msa_sparse_attn_bwd_workspace(int64_t N, int H_q, int H_kv, int d_h, int B_k, int k);
size_t msa_sparse_attn_bwd_workspace_min(int64_t N, int H_q, int H_kv, int d_h, int B_k, int k);
msa_status_t msa_sparse_attn_bwd(const void* q, const void* k, const void* v, const float* o,
                                 const float* lse, const void* dO, const int32_t* block_idx,
                                 int64_t N, int H_q, int H_kv, int d_h, int B_k, int k_sel,
                                 float scale, float* dq, float* dk, float* dv, void* ws,
                                 size_t ws_bytes, void* hip_stream);

/* ------------------------------------------------------------------ Packed sequences
 * Variable-length prefill: `batch` independent sequences packed along the token
 * axis, each with its own causal mask, block grid and local block (every position
 * in Eq. 6 - Eq. 8 counts from the start of its own sequence).  The pages train
 * on such packed documents; the arithmetic per sequence is that of the calls above.
 *   cu_seqlens int64 [batch + 1], device memory: cu[0] = 0, non-decreasing,
 *              cu[batch] = T; sequence s holds tokens cu[s] .. cu[s+1]-1 (length 0
 *              is allowed).  The host cannot check it; the kernels clamp what they
 *              read so that no access leaves the buffers: the index call reads
 *              sequence s as [clamp(cu[s], 0, T), clamp(cu[s+1], that, T)), the
 *              attention call first copies the table into its workspace with entry s
 *              replaced by the running maximum of cu[0..s] clamped into [0, T],
 *              entry 0 by 0 and entry batch by T.  A well-formed table is unchanged
 *              by both; for any other the results are unspecified but every read and
 *              write stays inside the caller's buffers.
 *   Tensors are those of the calls above with N replaced by T (rows stay global);
 *   block_idx entries are block numbers within the row's own sequence.
 *   Limits: ceil(T / B_k) + batch <= 8192, batch <= 65535.
 *
 * msa_index_topk_varlen — max_len (host) bounds every sequence length and sizes the
 *   launch; for a sequence longer than max_len some of its rows are left unwritten.
 * msa_sparse_attn_fwd_varlen — the workspace holds sequence tables built on the
 *   device from cu_seqlens, then the KV-outer buffers; sizes as for
 *   msa_sparse_attn_fwd.
 */
msa_status_t msa_index_topk_varlen(const void* q_idx, const void* k_idx, const int64_t* cu_seqlens,
                                   int batch, int64_t T, int64_t max_len, int H_kv, int d_idx,
                                   int B_k, int k, int32_t* block_idx, void* hip_stream);
size_t msa_sparse_attn_fwd_varlen_workspace(int64_t T, int batch, int H_q, int H_kv, int d_h,
                                            int B_k, int k);
size_t msa_sparse_attn_fwd_varlen_workspace_min(int64_t T, int batch, int H_q, int H_kv, int d_h,
                                                int B_k, int k);
msa_status_t msa_sparse_attn_fwd_varlen(const void* q, const void* k, const void* v,
                                        const int32_t* block_idx, const int64_t* cu_seqlens,
                                        int batch, int64_t T, int H_q, int H_kv, int d_h, int B_k,
                                        int k_sel, float scale, float* o, float* lse, void* ws,
                                        size_t ws_bytes, void* hip_stream);

/* ------------------------------------------------------------------ Decode
 * msa_decode — one new token per sequence against packed variable-length caches:
 * the decoding step whose wall-clock speedup the paper review page reports (section
 * 6, efficiency comparison, Figure 4; the reading notes page, result 3).  The
 * arithmetic is that of a single query row of the two-branch structure (reading
 * notes page, section 5.1: block scores, Top-k with the forced local block, then
 * softmax attention over the chosen blocks; paper review page, section 3, Eq. 6-8),
 * taken for the newest token only.  The new token's K/V and index key are already
 * the last cache entry of its sequence (position L_s - 1), so its local block is
 * block (L_s - 1) / B_k.  Every cached index key is scored once (an HBM-bound scan),
 * the best k blocks of each (sequence, group) are chosen, and the attention over
 * them is split across workgroups and merged by log-sum-exp.
 *   q            bf16 [batch, H_q, d_h];  q_idx  bf16 [batch, H_kv, d_idx]
 *   k_cache, v_cache bf16 [T, H_kv, d_h]; k_idx_cache bf16 [T, d_idx]
 *   cu_seqlens   int64 [batch + 1], device memory, cu[0] = 0, cu[s+1] - cu[s] = L_s;
 *                sequence s is read as [clamp(cu[s], 0, T), clamp(cu[s+1], that, T)),
 *                so a malformed table cannot read outside the caches (results are
 *                then unspecified)
 *   T            cached tokens (rows of the three caches), host
 *   max_len      host-side bound on every L_s (sizes the launch and workspace; a
 *                longer sequence is only scored over its first max_len tokens)
 *   block_idx    int32 [batch, H_kv, k]  out (as for msa_index_topk)
 *   o            fp32 [batch, H_q, d_h]; lse fp32 [batch, H_q]  out
 */
/* msa_decode_workspace — bytes of device workspace msa_decode needs for these shapes
 * (block scores of every cached block of every (sequence, group), then the partial
 * (m, l, o) of each split of the attention); it also sizes msa_decode_paged.  Returns
 * 0 for an unsupported shape.  Host-only. */
size_t msa_decode_workspace(int batch, int H_q, int H_kv, int d_h, int d_idx, int B_k, int k,
                            int64_t max_len);
msa_status_t msa_decode(const void* q, const void* q_idx, const void* k_cache, const void* v_cache,
                        const void* k_idx_cache, const int64_t* cu_seqlens, int batch, int64_t T,
                        int64_t max_len, int H_q, int H_kv, int d_h, int d_idx, int B_k, int k,
                        float scale, int32_t* block_idx, float* o, float* lse, void* ws,
                        size_t ws_bytes, void* hip_stream);

/* ------------------------------------------------------------------ Decode without allocation
 * msa_decode_noalloc — msa_decode for callers that cannot allocate device memory or
 * pass a workspace: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Arguments, outputs, results and errors are those of msa_decode
 * (bit-identical outputs for the same inputs); the workspace is the library's own
 * static device array of MSA_DECODE_NOALLOC_SCRATCH_BYTES (32 MiB), one per GPU,
 * which each GPU the library runs on holds until the process ends.  The call makes
 * no allocation of any kind.
 *   Limit: msa_decode_workspace() of the same shapes must be at most
 *   MSA_DECODE_NOALLOC_SCRATCH_BYTES (for example 64 sequences of up to 1M tokens with
 *   H_q = 64, H_kv = 8, k = 16 need 20 MiB; at 128K tokens, 6 MiB); larger shapes
 *   return MSA_ERR_WORKSPACE and launch nothing.
 *   Every call on a GPU uses that GPU's one array: calls that overlap in time on one
 *   GPU (different streams or host threads) race and give undefined results; calls
 *   ordered on one stream are safe.  Nothing in the array needs clearing between
 *   calls: each call writes every scratch value it reads.
 */
#define MSA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
msa_status_t msa_decode_noalloc(const void* q, const void* q_idx, const void* k_cache,
                                const void* v_cache, const void* k_idx_cache,
                                const int64_t* cu_seqlens, int batch, int64_t T, int64_t max_len,
                                int H_q, int H_kv, int d_h, int d_idx, int B_k, int k, float scale,
                                int32_t* block_idx, float* o, float* lse, void* hip_stream);

/* ------------------------------------------------------------------ Paged FP8 decode
 * msa_decode_paged — msa_decode over a paged cache whose K/V are FP8 (the open
 * interface's paged FP8 decode path, reading notes, section 5.4).  Pages hold B_k
 * tokens; token j of sequence s is row j % B_k of page block_table[s][j / B_k].
 *   k_pages, v_pages  uint8 [P, B_k, H_kv, d_h]  OCP FP8 E4M3 codes; the cached
 *                     K = k_scale * value, V = v_scale * value (per-tensor scales)
 *   k_idx_pages       bf16 [P, B_k, d_idx]       index keys (kept at bf16: they
 *                     decide the selection)
 *   block_table       int32 [batch, max_blocks], device; entries for blocks
 *                     0 .. ceil(L_s / B_k) - 1 must be page numbers in [0, P), the
 *                     rest are never read
 *   num_pages         P, the pages of the three page arrays (>= 1), host
 *   seqlens           int64 [batch], device: L_s (the new token is position L_s - 1)
 *   The kernels read L_s clamped into [0, max_blocks * B_k] and every page number
 *   clamped into [0, P - 1], so malformed tables cannot read outside the buffers
 *   (results are then unspecified).
 *   max_len           host-side bound on every L_s, as for msa_decode
 * Other arguments and outputs as msa_decode; the workspace size is
 * msa_decode_workspace() of the same shapes.  FP8 values are widened to bf16
 * exactly; the K scale multiplies the scores and the V scale the output.
 */
msa_status_t msa_decode_paged(const void* q, const void* q_idx, const void* k_pages,
                              const void* v_pages, float k_scale, float v_scale,
                              const void* k_idx_pages, const int32_t* block_table,
                              int64_t max_blocks, int64_t num_pages, const int64_t* seqlens,
                              int batch, int64_t max_len, int H_q, int H_kv, int d_h, int d_idx,
                              int B_k,
                              int k, float scale, int32_t* block_idx, float* o, float* lse,
                              void* ws, size_t ws_bytes, void* hip_stream);

/* ------------------------------------------------------------------ Split entry points
 * The pages' open interface separates a pass that emits per-block max scores from
 * the Top-k select (reading notes page, section 5.4).  These two calls expose the
 * same split for testing; msa_index_topk fuses them.
 *
 * msa_index_block_scores — Eq. 6: M fp32 [N, H_kv, B] with B = ceil(N / B_k),
 *   M[i][r][b] = max_{j in block b, j <= i} <q_idx[i,r], k_idx[j]> / sqrt(d_idx);
 *   -inf where block b has no visible token.
 * msa_topk_from_scores — Eq. 7 on given scores: M fp32 [N, H_kv, B] (row stride B,
 *   B >= ceil(N / B_k)); only M[i][r][b] for b < i / B_k is read.  Output as for
 *   msa_index_topk.  -inf scores rank below every finite one (ties to the lower
 *   block as usual); with NaN scores the selection is unspecified.
 */
msa_status_t msa_index_block_scores(const void* q_idx, const void* k_idx, int64_t N, int H_kv,
                                    int d_idx, int B_k, float* M, void* hip_stream);
msa_status_t msa_topk_from_scores(const float* M, int64_t N, int H_kv, int64_t B, int B_k, int k,
                                  int32_t* block_idx, void* hip_stream);

/* Measurement hook, not part of the method: while set, each msa_sparse_attn_fwd or
 * msa_sparse_attn_fwd_varlen call made on this host thread records, on its stream,
 * for its query window w < n / 4: events[4w] before the inverse index (counts,
 * scan, scatter), events[4w+1] before the KV-outer phase-1 kernel, events[4w+2]
 * before the combine and events[4w+3] after it.  Later windows record nothing
 * (msa_sparse_attn_fwd_windows gives a call's window count).
 *   events  n hipEvent_t handles owned by the caller; they must stay valid while set.
 *   n       4 * m with 1 <= m <= 1024 to set, 0 to clear (events is then ignored).
 * Returns MSA_ERR_INVALID_ARG for any other n or a null handle (the previous setting
 * is kept).  Host-only; no device work. */
msa_status_t msa_set_profile_events(void* const* events, int n);

/* msa_set_profile_clock — measurement hook for the load balance of the persistent-grid
 * kernels (the pages balance variable work with a persistent grid and an atomic
 * counter: paper review page, section 4; here eight per-XCD atomic item counters
 * play that part).  While set,
 * the KV-outer phase-1 kernel of the first query window of every later
 * msa_sparse_attn_fwd / _varlen call on this host thread, and the main kernel of the
 * first query window of every later msa_sparse_attn_bwd call, store for each workgroup
 * w the GPU's constant-rate clock (100 MHz) at its start in clock[2w] and after its
 * last item in clock[2w + 1].  A launch whose grid needs more than `slots` entries
 * (at most 2 * (2 * CUs + 8)) records nothing.
 *   clock  device buffer of `slots` uint64, owned by the caller, valid while set.
 *   slots  its length; 0 clears the hook (clock is then ignored).
 * Returns MSA_ERR_INVALID_ARG for a negative size or a null / misaligned buffer.
 * Host-only; no device work. */
msa_status_t msa_set_profile_clock(uint64_t* clock, int64_t slots);

#ifdef __cplusplus
}
#endif
#endif /* MSA_H */
