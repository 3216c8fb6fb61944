// Host-side launchers of the MSA kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace msa {

// Shapes of the fast path (head dim, index head dim, keys per block).
constexpr int kHeadDim = 128;
constexpr int kIndexDim = 64;
constexpr int kBlockKeys = 128;

// Chunks (of 128 MFMA rows) per work item of the KV-outer kernel.
constexpr int kItemChunks = 16;
// Pairs per backward work item (its pair list sits in LDS).  A longer item writes
// fewer fp32 dK/dV partial blocks (128 KB each) and stages its K/V block fewer
// times; measured at 128K: 256 pairs 44.7-45.9 ms, 512 43.3, 1024 42.7-43.5, 2048
// 42.7-42.9 (longer items lengthen the schedule's tail).
constexpr int kBwdItemPairs = 1024;

// Distance (in int32) between the per-XCD item counters of a workspace; a workspace
// holds kItemCounterSets sets of eight (one per persistent launch over its items).
constexpr int kItemCounterStride = 64;
constexpr int kItemCounterSets = 2;

// Floats per (query, group, slot) partial of the KL pass.
constexpr int kKlPart = 8;

struct AttnWorkspace {
  size_t counts, tsum, cursor, n_items, ctr, items, pairs, opart, lpart, lidx, lfirst, tcount, total;
  int64_t max_items;
  int item_q;  // queries per work item
  int64_t WQ;  // queries per q-locality window
  int nW;      // q-locality windows per call window
};

struct DecodeWorkspace {
  size_t M, opart, lpart, total;
};

// bk: keys per block, 64 or 128.
hipError_t launch_index_topk(const uint16_t* q_idx, const uint16_t* k_idx, int64_t N, int H_kv, int k,
                             int32_t* block_idx, const int64_t* cu, int batch, int64_t T, int bk, int num_cus,
                             hipStream_t stream);
hipError_t launch_index_block_scores(const uint16_t* q_idx, const uint16_t* k_idx, int64_t N, int H_kv, int bk,
                                     float* M, hipStream_t stream);
hipError_t launch_topk_from_scores(const float* M, int64_t N, int H_kv, int64_t B, int k, int bk,
                                   int32_t* block_idx, hipStream_t stream);

// Packed sequences of a varlen call: cu == nullptr means one sequence [0, N).
// bstart[s] is the first global block of sequence s (blocks of all sequences are
// numbered consecutively; bstart[batch] = their count), seq_tok[t] the sequence of
// token t and seq_blk[gb] the sequence of global block gb.
struct SeqInfo {
  const int64_t* cu = nullptr;
  const int32_t* bstart = nullptr;
  const int32_t* seq_tok = nullptr;
  const int32_t* seq_blk = nullptr;
};
struct SeqTables {
  size_t cu, bstart, seq_tok, seq_blk, total;
};
// Workspace bytes of the tables for T tokens in `batch` sequences with at most Bt
// global blocks (0 for a single sequence).
SeqTables seq_tables_layout(int64_t T, int batch, int64_t Bt);
// Builds the tables from the caller's offsets cu[0..batch]: first a sanitised copy of
// the offsets (region S.cu; every later kernel reads that copy), then the block starts
// and the per-token and per-block sequence numbers.
hipError_t launch_seq_tables(const int64_t* cu, int batch, int64_t T, int bk, uint8_t* ws, const SeqTables& S,
                             hipStream_t stream);

// B: the list stride in blocks (the block count, or for several sequences an upper
// bound of the global block count).
// Inverse index of one query window (lists, item table, pairs) in the workspace
// regions of L; lfirst (lists entries, may be null) receives each list's first item.
// ordered: each list's pairs in (query, slot) order, decided by no atomic (needs the
// workspace's per-tile counts, laid out for kPartsBwd); otherwise the order within a
// list follows the scatter's atomic counters.
hipError_t launch_inverse_index(const int32_t* block_idx, int64_t B, const SeqInfo& si, int bsh, int H_kv, int kk,
                                int64_t w0, int64_t W, uint8_t* ws, const AttnWorkspace& L, hipStream_t stream,
                                int32_t* lfirst = nullptr, bool ordered = false);

// What the per-pair and per-item buffers hold: the attention's partial rows, the KL
// pass's kKlPart floats per pair, or the backward's fp32 dQ rows per pair plus a
// dK/dV block per item (and each list's first item).
enum PartKind { kPartsAttn = 0, kPartsKl = 1, kPartsBwd = 2 };
AttnWorkspace attn_workspace_layout(int64_t W, int H_q, int H_kv, int kk, int64_t B, int parts = kPartsAttn);
// bk: keys per block, 64 or 128.
hipError_t launch_sparse_attn_window(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const int32_t* block_idx, int64_t N, int64_t B, const SeqInfo& si, int bk,
                                     int H_q, int H_kv, int kk, float scale, int64_t w0, int64_t W, int num_cus,
                                     float* o, float* lse, uint8_t* ws, const AttnWorkspace& L, hipStream_t stream,
                                     const hipEvent_t* events,  // 4 phase events or null
                                     uint64_t* clk,             // per-workgroup clock of phase 1, or null
                                     const uint16_t* q_idx = nullptr, const uint16_t* k_idx = nullptr,
                                     float* lse_idx = nullptr);  // LSE_idx [N, H_kv] when set

// KL alignment pass over one query window (single sequence of N tokens): per
// (query, group) kl and lse_idx.  launch_kl_loss then reduces kl [n] to its mean in
// a fixed order (partial: kKlLossParts doubles of workspace).
constexpr int kKlLossParts = 256;
hipError_t launch_sparse_kl_window(const uint16_t* q, const uint16_t* k, const uint16_t* q_idx,
                                   const uint16_t* k_idx, const float* lse, const int32_t* block_idx, int64_t N,
                                   int64_t B, int bk, int H_q, int H_kv, int kk, float scale, int64_t w0, int64_t W,
                                   int num_cus, const float* lse_idx_in,  // given LSE_idx, or null
                                   float* kl, float* lse_idx, uint8_t* ws, const AttnWorkspace& L,
                                   hipStream_t stream);
hipError_t launch_kl_loss(const float* kl, int64_t n, double* partial, float* loss, hipStream_t stream);

// Backward of the Main Branch (single sequence, B_k = 64 or 128, G <= 32): D = <dO, o> per
// (query, head) and zeroed dk / dv, then per query window the KV-outer pass and the
// reductions of its dQ rows and dK/dV blocks.
hipError_t launch_bwd_prepare(const uint16_t* dO, const float* o, int64_t rows, float* D, float* dk, float* dv,
                              int64_t kv_elems, hipStream_t stream);
hipError_t launch_bwd_window(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dO,
                             const float* lse, const float* D, const int32_t* block_idx, int64_t N, int64_t B,
                             int bk, int H_q, int H_kv, int kk, float scale, int64_t w0, int64_t W, int num_cus,
                             float* dq, float* dk, float* dv, uint8_t* ws, const AttnWorkspace& L,
                             hipStream_t stream, uint64_t* clk);  // per-workgroup clock, or null

DecodeWorkspace decode_workspace_layout(int batch, int H_q, int H_kv, int kk, int64_t Bmax);
hipError_t launch_decode(const uint16_t* q, const uint16_t* q_idx, const uint16_t* k_cache,
                         const uint16_t* v_cache, const uint16_t* k_idx_cache, const int64_t* cu, int batch,
                         int64_t T, int64_t Bmax, int bk, int H_q, int H_kv, int kk, float scale, int32_t* block_idx, float* o,
                         float* lse, uint8_t* ws, const DecodeWorkspace& L, hipStream_t stream);
// Paged caches: FP8 E4M3 K/V pages and bf16 index-key pages of bk tokens (64 or 128).
hipError_t launch_decode_paged(const uint16_t* q, const uint16_t* q_idx, const uint8_t* k_pages,
                               const uint8_t* v_pages, float k_scale, float v_scale, const uint16_t* kidx_pages,
                               const int32_t* block_table, int64_t max_blocks, int64_t num_pages,
                               const int64_t* seqlens, int batch, int64_t Bmax, int bk, int H_q, int H_kv, int kk, float scale, int32_t* block_idx,
                               float* o, float* lse, uint8_t* ws, const DecodeWorkspace& L, hipStream_t stream);

}  // namespace msa
