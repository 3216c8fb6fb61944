// Index Branch kernels: index scoring on MFMA with a fused causal mask and block
// max-pool, and the exp-free Top-k with the forced local block.
//
// Method: page "MiniMax Sparse Attention (MSA)" paper review, section 3, Eq. 6
// (token scores and causal block max-pool) and Eq. 7 (Top-k, local block kept);
// reading notes page, section 5.1.1 (local block takes one slot, invisible
// tokens are -inf) and section 5.4 (selection on raw scores, no softmax).
//
// Layout of the work: the (query, group) pairs are flattened into "columns"
// c = i * H_kv + r (the natural row order of q_idx and block_idx).  A workgroup
// owns a run of consecutive columns and sweeps the 128-key tiles 0..b_last in
// order; a tile is one block (B_k = 128) or two (B_k = 64).  Each tile (128 keys x
// 64 dims, 16 KB) is staged once in LDS and shared by every wave.  A wave computes S^T = K_block * Q^T with 32x32x16 bf16 MFMAs, so
// each lane owns one column and holds 16 of the 32 keys of a tile: the max-pool is
// a per-lane running max plus one swap between the two lane halves.  The block
// score then goes straight into a per-lane Top-L register list (Top-k fused) or,
// for the split entry point, to memory.  The token scores never leave registers.
#include "msa_device.h"
#include "msa_kernels.h"
#include "table_clamp.h"

namespace msa {

namespace {

constexpr int kIdxWaves = 8;
constexpr int kIdxThreads = kIdxWaves * kWave;
constexpr int kIdxBlocksPerCU = 8 / kIdxWaves;     // two waves per SIMD

// Stage key tile b of k_idx (128 keys) into LDS: 128 rows x 8 chunks of 16 B, chunk c
// of row j stored at chunk position c ^ ((j >> 1) & 7): the 16 rows a 16-lane LDS
// pass reads then fall on 16 different 16-byte bank groups.  The 16-byte global ->
// LDS loads write lane l's 16 bytes at the instruction's LDS base + 16 l (measured on
// the GPU with an in-bounds probe), so each wave instruction fills 8 rows (1 KB) and
// a lane fetches the global chunk that belongs at its LDS position.  Keys past the
// end read the last key (their scores are masked: no query sees them).
constexpr int kIdxDmaPerWave = 16 / kIdxWaves;  // 1 KB instructions per wave per tile
constexpr unsigned kWaitVmcnt0 = 0x0F70;        // s_waitcnt vmcnt(0), other counters free

__device__ __forceinline__ void idx_dma_block(const uint16_t* __restrict__ k_idx, int64_t N, int64_t b, int wave,
                                              int lane, uint8_t* buf) {
#pragma unroll
  for (int t = 0; t < kIdxDmaPerWave; ++t) {
    const int m = wave + kIdxWaves * t;  // rows 8m .. 8m+7 (uniform per wave)
    const int key = 8 * m + (lane >> 3);
    const int c = (lane & 7) ^ ((key >> 1) & 7);
    int64_t j = b * kBk + key;
    j = j < N ? j : N - 1;
    __builtin_amdgcn_global_load_lds(k_idx + j * kDidx + c * 8, buf + m * 1024, 16, 0, 0);
  }
}

// Block maxima of one staged key block for the lane's CT column tiles (raw dot
// products; the 1/sqrt(d_idx) scale is applied by the caller when needed).
// The 4 x CT output tiles are software-pipelined over two accumulators: the four
// MFMAs of tile j+1 are issued before tile j is max-reduced, so the VALU reduction
// of one tile runs under the matrix work of the next.
template <bool MASK>
__device__ __forceinline__ void idx_tile_reduce(const f32x16_t& acc, int qi, int64_t b, int kt, int h, float& bmax) {
  if constexpr (MASK) {
    // key b*128 + kt*32 + 8*(v/4) + 4h + v%4 is visible iff its offset <= lim
    int64_t lim64 = (int64_t)qi - (b * kBk + kt * 32 + 4 * h);
    lim64 = lim64 < -1 ? -1 : (lim64 > 64 ? 64 : lim64);
    const int lim = (int)lim64;
#pragma unroll
    for (int v = 0; v < 16; ++v) bmax = fmaxf(bmax, (8 * (v >> 2) + (v & 3)) <= lim ? acc[v] : -__builtin_inff());
  } else {
#pragma unroll
    for (int v = 0; v < 16; ++v) bmax = fmaxf(bmax, acc[v]);
  }
}

// NS blocks per staged tile (1 for B_k = 128, 2 for B_k = 64): 32-key MFMA tile kt
// belongs to block kt / (4 / NS) of the staged tile.  MASK: some key of the tile
// lies past some column's query (the causal mask is applied per key); decided once
// per staged tile, so the unmasked sweep carries no per-tile branch.
template <int CT, int NS, bool MASK>
__device__ __forceinline__ void idx_block_max(const uint8_t* buf, const uint4 (&qop)[CT][4], const int (&qi)[CT],
                                              int64_t b, int h, int l32, float (&bmax)[CT][NS]) {
  constexpr int kTiles = 4 * CT;
  constexpr int kPerBlock = 4 / NS;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
    for (int u = 0; u < NS; ++u) bmax[ct][u] = -__builtin_inff();
  }
  u32x4_t a[4];
  f32x16_t acc[2];
  // Raised wave priority over the matrix section: of the two waves of a SIMD, the
  // one issuing MFMAs keeps the issue slot (measured: 2% less time).
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int j = 0; j < kTiles; ++j) {
    const int kt = j / CT, ct = j % CT;
    if (ct == 0) {
      const int key = kt * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int c = ks * 2 + h;
        a[ks] = *reinterpret_cast<const u32x4_t*>(buf + key * 128 + ((c ^ ((key >> 1) & 7)) << 4));
      }
    }
    acc[j & 1] = f32x16_t{};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) acc[j & 1] = mfma_32x32x16(as_bf16x8(a[ks]), as_bf16x8(qop[ct][ks]), acc[j & 1]);
    if (j > 0) {
      const int pj = j - 1, pkt = pj / CT, pct = pj % CT;
      idx_tile_reduce<MASK>(acc[pj & 1], qi[pct], b, pkt, h, bmax[pct][pkt / kPerBlock]);
    }
    // Each MFMA of tile j is followed by a share of tile j-1's reduction, so the
    // VALU work issues while the matrix unit runs (left to itself the compiler
    // paired two tiles' MFMAs and then reduced both, with no overlap in the wave).
    if (ct == 0) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    if (j == 0) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, MASK ? 12 : 2, 0);
      }
    }
  }
  {
    constexpr int pj = kTiles - 1, pkt = pj / CT, pct = pj % CT;
    idx_tile_reduce<MASK>(acc[pj & 1], qi[pct], b, pkt, h, bmax[pct][pkt / kPerBlock]);
  }
  __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
    for (int u = 0; u < NS; ++u) bmax[ct][u] = fmaxf(bmax[ct][u], __shfl_xor(bmax[ct][u], 32));
  }
}

template <int CT, int NS>
__device__ __forceinline__ void idx_block_max(const uint8_t* buf, const uint4 (&qop)[CT][4], const int (&qi)[CT],
                                              int64_t b, bool need_mask, int h, int l32, float (&bmax)[CT][NS]) {
  if (need_mask)
    idx_block_max<CT, NS, true>(buf, qop, qi, b, h, l32, bmax);
  else
    idx_block_max<CT, NS, false>(buf, qop, qi, b, h, l32, bmax);
}

// LIST: register list length (>= k-1); CT: 32-column tiles per wave (even).
// WRITE_M: emit block scores M[c][b] (scaled) instead of selecting.
//
// Selection: staged tiles are swept in pairs (b, b+1).  After a pair both lane halves
// hold every block maximum of all CT columns of the lane; the lower half keeps the
// Top-k lists of the first CT/2 columns and offers them both tiles' blocks, the upper
// half those of the other CT/2 columns, so each column has one list and needs no
// merge at the end.
// Sequences: with cu == nullptr the call is one sequence of N tokens; otherwise
// cu[0..batch] (device) are the packed sequence offsets of T tokens, grid.y is the
// sequence and grid.x the column tile within it (tiles past the sequence's end exit).
// The span read from cu is clamped into [0, T) and its length to N_all (the host's
// bound on every length), so a malformed table stays inside the buffers.  Every
// position below (queries, blocks, keys) is relative to the sequence start j0;
// columns and output rows are global.
template <int LIST, int CT, bool WRITE_M, int BK>
__global__ __launch_bounds__(kIdxThreads, kIdxBlocksPerCU) void index_topk_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx_all, int64_t N_all, int H_kv,
    int k, int64_t B, int32_t* __restrict__ block_idx, float* __restrict__ M, const int64_t* __restrict__ cu,
    int64_t T, uint32_t imask) {
  constexpr int NS = kBk / BK;  // blocks per staged 128-key tile
  constexpr int kColsPerWave = 32 * CT;
  constexpr int kCols = kIdxWaves * kColsPerWave;
  constexpr int kBlkBytes = kBk * kDidx * 2;
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][2][kBlkBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: kept in scalar registers
  const int h = lane >> 5, l32 = lane & 31;
  const PackedSpan span = cu ? packed_span(cu[blockIdx.y], cu[blockIdx.y + 1], T) : PackedSpan{0, N_all};
  const int64_t j0 = span.start;
  const int64_t N = span.len < N_all ? span.len : N_all;  // tokens of this sequence
  const uint16_t* __restrict__ k_idx = k_idx_all + j0 * kDidx;
  const int64_t total = N * H_kv;                          // columns of this sequence
  const int64_t ntiles = (total + kCols - 1) / kCols;
  if ((int64_t)blockIdx.x >= ntiles) return;
  // Longest sweeps (largest query positions) are dispatched first.
  const int64_t tile = ntiles - 1 - blockIdx.x;
  const int64_t c0 = tile * kCols;
  const int64_t c_end = (c0 + kCols < total ? c0 + kCols : total);
  const int64_t b_last = ((c_end - 1) / H_kv) / kBk;
  const int64_t wave_c0 = c0 + wave * kColsPerWave;
  const int64_t i_min_wave = wave_c0 / H_kv;
  const int64_t gcol0 = j0 * H_kv;  // global column of the sequence's first column

  static_assert(CT % 2 == 0, "the lane halves keep the lists of CT / 2 columns each");
  constexpr int CH = CT / 2;
  int qi[CT];  // query position of the lane's column in tile ct (-1 past the end)
  uint4 qop[CT][4];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int64_t c = wave_c0 + ct * 32 + l32;
    const bool ok = c < total;
    qi[ct] = ok ? (int)(c / H_kv) : -1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qop[ct][ks] = ok ? *reinterpret_cast<const uint4*>(q_idx + (gcol0 + c) * kDidx + ks * 16 + 8 * h)
                       : make_uint4(0, 0, 0, 0);
  }

  // This lane half's columns: tiles h * CH .. h * CH + CH - 1; their local blocks.
  KeyList<LIST> list[CH];
  int bloc[CH];
  if constexpr (!WRITE_M) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      list[c].init();
      // The column's query, recomputed rather than taken from qi[] by the lane's half
      // (an index the compiler would lower to a private-memory array).
      const int64_t col = wave_c0 + (h * CH + c) * 32 + l32;
      bloc[c] = col < total ? (int)(col / H_kv) / BK : -1;
    }
  }

  // Key tiles go straight from global memory to LDS (no registers), one step ahead:
  // tiles b+2, b+3 are loaded into the other buffer pair while b, b+1 are computed.
  idx_dma_block(k_idx, N, 0, wave, lane, kbuf[0][0]);
  if (b_last >= 1) idx_dma_block(k_idx, N, 1, wave, lane, kbuf[0][1]);
  int step = 0;
  for (int64_t b = 0; b <= b_last; b += 2, ++step) {
    const bool two = b + 1 <= b_last;
    uint8_t* buf0 = kbuf[step & 1][0];
    uint8_t* buf1 = kbuf[step & 1][1];
    // This wave's loads of the pair have landed; after the barrier everyone's have,
    // and everyone has finished reading the other pair (the previous step's).
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    __syncthreads();
    if (b + 2 <= b_last) idx_dma_block(k_idx, N, b + 2, wave, lane, kbuf[(step + 1) & 1][0]);
    if (b + 3 <= b_last) idx_dma_block(k_idx, N, b + 3, wave, lane, kbuf[(step + 1) & 1][1]);

    float m0[CT][NS], m1[CT][NS];
    idx_block_max<CT, NS>(buf0, qop, qi, b, b * kBk + (kBk - 1) > i_min_wave, h, l32, m0);
    if (two) {
      idx_block_max<CT, NS>(buf1, qop, qi, b + 1, (b + 1) * kBk + (kBk - 1) > i_min_wave, h, l32, m1);
    } else {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
        for (int u = 0; u < NS; ++u) m1[ct][u] = -__builtin_inff();
      }
    }
    if constexpr (WRITE_M) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
          // block (b + h) * NS + u: this lane half's tile
          const int64_t blk = (b + h) * NS + u;
          const float x = h ? m1[ct][u] : m0[ct][u];
          if (qi[ct] >= 0 && (h == 0 || two) && blk < B)
            M[(gcol0 + wave_c0 + ct * 32 + l32) * B + blk] = x * 0.125f;  // 1/sqrt(64), exact
        }
      }
    } else {
      // Blocks before the local one compete (key 0 offers nothing); the local block
      // is forced when the row is written.  A block past b_last has no visible key
      // for any column, so its -inf maximum is never offered.
#pragma unroll
      for (int c = 0; c < CH; ++c) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
          const int blk0 = (int)b * NS + u, blk1 = (int)(b + 1) * NS + u;
          const float x0 = h ? m0[CH + c][u] : m0[c][u];
          const float x1 = h ? m1[CH + c][u] : m1[c][u];
          list[c].offer(blk0 < bloc[c] ? block_key(x0, blk0, imask) : 0u);
          list[c].offer(blk1 < bloc[c] ? block_key(x1, blk1, imask) : 0u);
        }
      }
    }
  }

  if constexpr (!WRITE_M) {
    // The lane's number, taken afresh (not kept live across the sweep, where every
    // register is in use).
    const int lid = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (bloc[c] < 0) continue;
      int cand[LIST + 1];
#pragma unroll
      for (int j = 0; j < LIST; ++j) {
        const int blk = block_key_block(list[c].k[j], imask);
        cand[j] = (j < k - 1 && blk >= 0) ? blk : 0x7fffffff;
      }
      cand[LIST] = 0x7fffffff;
      int32_t out[LIST + 1];
      write_selection<LIST + 1>(cand, k, bloc[c], out);
      int32_t* row = block_idx + (gcol0 + wave_c0 + ((lid >> 5) * CH + c) * 32 + (lid & 31)) * k;
#pragma unroll
      for (int t = 0; t <= LIST; ++t) {
        if (t < k) row[t] = out[t];
      }
    }
  }
}

// Top-k of given block scores (the split form of the selection), one wave per
// (query, group) row, four rows per workgroup.  Block b < b_loc of the row has the
// 64-bit key rank_key(score, b): score first, then the lower block.  The k-1 best
// keys are found without sorting the row:
//  1. lane l takes blocks l, l + 64, ... (coalesced across the wave; up to 32 chunks
//     of 64 stay in registers, longer rows are streamed twice) and keeps its best key.  The (k-1)-th best of
//     the 64 lane bests, t0, is reached by k-1 distinct blocks, so every one of the
//     row's k-1 best keys is >= t0;
//  2. the blocks with key >= t0 are compacted into LDS in block order (ballot and
//     lane-prefix counts); only the k-1 lanes whose best reaches t0 contribute;
//  3. a candidate is kept iff fewer than k-1 candidates beat it; the kept ones are
//     written in candidate order, which is ascending block order, and the local
//     block b_loc (larger than all) follows.
// A row with more than kTfsCap candidates (a few lanes owning most of the best
// blocks; impossible below 17 chunks) takes k-1 rounds of wave arg-max instead.
constexpr int kTfsCap = 512;

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int lane_prefix(uint64_t bal) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
}

// Step 1's threshold t0: the lane best that exactly kk-1 lane bests exceed
// (nonzero keys are distinct and at least kk+1 lanes hold one).  s_lb: the wave's
// 64-entry LDS table.
__device__ __forceinline__ uint64_t tfs_threshold(uint64_t lbest, uint64_t* s_lb, int lane, int kk) {
  s_lb[lane] = lbest;
  wave_lds_sync();
  int above = 0;
#pragma unroll 8
  for (int l = 0; l < 64; ++l) above += s_lb[l] > lbest;
  const uint64_t who = __ballot(above == kk - 1);
  const int wl = __builtin_ctzll(who);
  return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(lbest >> 32), wl) << 32) |
         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)lbest, wl);
}

// Step 3 over C <= kTfsCap candidates s_c[0..C) in block order: keep those that fewer
// than kk others beat, in candidate order, then the local block bl.
__device__ __forceinline__ void tfs_write_kept(const uint64_t* s_c, int C, int kk, int lane, int bl,
                                               int32_t* orow) {
  int S = 0;
  for (int m0 = 0; m0 < C; m0 += 64) {
    const int ci = m0 + lane;
    const uint64_t key = ci < C ? s_c[ci] : ~0ull;
    int beat = 0;
    for (int cj = 0; cj < C; ++cj) beat += s_c[cj] > key;
    const bool keep = ci < C && beat < kk;
    const uint64_t bal = __ballot(keep);
    if (keep) orow[S + lane_prefix(bal)] = rank_key_block(key);
    S += __popcll(bal);
  }
  if (lane == 0) orow[S] = bl;  // S == kk
}

// The overflow path: kk rounds of wave arg-max, each below the previous round's key
// (best_below(prev) returns the lane's best key below prev); lane t keeps round t's
// block, then the kk blocks are placed by their rank.  s_c: the wave's candidate area.
template <typename F>
__device__ __forceinline__ void tfs_rounds(F&& best_below, uint64_t* s_c, int kk, int lane, int bl, int32_t* orow) {
  uint64_t prev = ~0ull;
  int mine = 0x7fffffff;
  for (int t = 0; t < kk; ++t) {
    prev = wave_max_u64(best_below(prev));
    if (lane == t) mine = rank_key_block(prev);
  }
  wave_lds_sync();
  s_c[lane] = (uint64_t)(uint32_t)mine;
  wave_lds_sync();
  if (lane < kk) {
    int pos = 0;
    for (int t = 0; t < kk; ++t) pos += (int)s_c[t] < mine;
    orow[pos] = mine;
  }
  if (lane == 0) orow[kk] = bl;
}

// Rows that select everything or only the local block; true when the row is done.
__device__ __forceinline__ bool tfs_trivial(int kk, int bl, int k, int lane, int32_t* orow) {
  if (kk == 0) {
    if (lane == 0) orow[0] = bl;
    return true;
  }
  if (bl <= kk) {  // every causal block is chosen
    for (int t = lane; t < k; t += 64) orow[t] = t <= bl ? t : -1;
    return true;
  }
  return false;
}

template <int R>
__global__ __launch_bounds__(256) void topk_from_scores_kernel(const float* __restrict__ M, int64_t N,
                                                                int H_kv, int64_t B, int k, int bk,
                                                                int32_t* __restrict__ block_idx) {
  __shared__ uint64_t s_cand[4][kTfsCap];
  __shared__ uint64_t s_lbest[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t c = (int64_t)blockIdx.x * 4 + w;
  if (c >= N * H_kv) return;  // whole waves
  const int bl = (int)((c / H_kv) / bk);
  const int kk = k - 1;  // blocks chosen besides the local one
  const float* row = M + c * B;
  int32_t* orow = block_idx + c * k;
  if (tfs_trivial(kk, bl, k, lane, orow)) return;
  const int nch = (bl + 63) >> 6;  // >= 1; kk < bl blocks and kk < 64 lanes hold one

  // 1. The row's scores, chunk j in x[j] (nch <= R); each lane's best key.
  float x[R];
  uint64_t lbest = 0;
#pragma unroll
  for (int g = 0; g < R; g += 16) {
    if (g < nch) {
#pragma unroll
      for (int j = g; j < g + 16; ++j) {
        const int b = j * 64 + lane;
        x[j] = row[b < bl ? b : 0];
      }
#pragma unroll
      for (int j = g; j < g + 16; ++j) {
        const int b = j * 64 + lane;
        const uint64_t key = b < bl ? rank_key(x[j], b) : 0ull;
        lbest = key > lbest ? key : lbest;
      }
    }
  }
  const uint64_t t0 = tfs_threshold(lbest, s_lbest[w], lane, kk);

  // 2. Candidates (key >= t0) in block order.
  int C = 0;
  auto offer = [&](uint64_t key) {
    const bool p = key >= t0;
    const uint64_t bal = __ballot(p);
    const int pos = C + lane_prefix(bal);
    if (p && pos < kTfsCap) s_cand[w][pos] = key;
    C += __popcll(bal);
  };
#pragma unroll
  for (int j = 0; j < R; ++j) {
    if (j < nch) {
      const int b = j * 64 + lane;
      offer(b < bl ? rank_key(x[j], b) : 0ull);
    }
  }
  wave_lds_sync();
  if (C <= kTfsCap) {
    tfs_write_kept(s_cand[w], C, kk, lane, bl, orow);  // 3.
  } else {
    tfs_rounds(
        [&](uint64_t prev) {
          uint64_t best = 0;
#pragma unroll
          for (int j = 0; j < R; ++j) {
            if (j < nch) {
              const int b = j * 64 + lane;
              const uint64_t key = b < bl ? rank_key(x[j], b) : 0ull;
              best = (key < prev && key > best) ? key : best;
            }
          }
          return best;
        },
        s_cand[w], kk, lane, bl, orow);
  }
}

// Rows of more than 32 chunks: the same three steps, with the row streamed from
// memory in groups of kTfsGroup chunks instead of held in registers (which at 64 or
// 128 chunks left two or one waves per SIMD): one sweep for the lane bests, a second
// for the candidates (mostly re-read from the L2), and for the overflow path one per
// round.  Measured at 512K rows: 4096 blocks 2.45 -> 1.45-1.52 ms, 8192 blocks (k =
// 32) 8.78 -> 2.63-2.83 ms, the same selections.
constexpr int kTfsGroup = 32;

__global__ __launch_bounds__(256) void topk_from_scores_long_kernel(const float* __restrict__ M, int64_t N,
                                                                     int H_kv, int64_t B, int k, int bk,
                                                                     int32_t* __restrict__ block_idx) {
  __shared__ uint64_t s_cand[4][kTfsCap];
  __shared__ uint64_t s_lbest[4][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t c = (int64_t)blockIdx.x * 4 + w;
  if (c >= N * H_kv) return;  // whole waves
  const int bl = (int)((c / H_kv) / bk);
  const int kk = k - 1;
  const float* row = M + c * B;
  int32_t* orow = block_idx + c * k;
  if (tfs_trivial(kk, bl, k, lane, orow)) return;
  const int nch = (bl + 63) >> 6;

  // fn(key) for every chunk of the row in block order (lane l: blocks l, l + 64, ...;
  // a block at or past bl offers key 0).  Each group's loads are issued together.
  auto sweep = [&](auto&& fn) {
    for (int g0 = 0; g0 < nch; g0 += kTfsGroup) {
      float x[kTfsGroup];
#pragma unroll
      for (int j = 0; j < kTfsGroup; ++j) {
        const int b = (g0 + j) * 64 + lane;
        x[j] = g0 + j < nch ? row[b < bl ? b : 0] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < kTfsGroup; ++j) {
        if (g0 + j < nch) {
          const int b = (g0 + j) * 64 + lane;
          fn(b < bl ? rank_key(x[j], b) : 0ull);
        }
      }
    }
  };
  uint64_t lbest = 0;
  sweep([&](uint64_t key) { lbest = key > lbest ? key : lbest; });
  const uint64_t t0 = tfs_threshold(lbest, s_lbest[w], lane, kk);
  int C = 0;
  sweep([&](uint64_t key) {
    const bool p = key >= t0;
    const uint64_t bal = __ballot(p);
    const int pos = C + lane_prefix(bal);
    if (p && pos < kTfsCap) s_cand[w][pos] = key;
    C += __popcll(bal);
  });
  wave_lds_sync();
  if (C <= kTfsCap) {
    tfs_write_kept(s_cand[w], C, kk, lane, bl, orow);
  } else {
    tfs_rounds(
        [&](uint64_t prev) {
          uint64_t best = 0;
          sweep([&](uint64_t key) { best = (key < prev && key > best) ? key : best; });
          return best;
        },
        s_cand[w], kk, lane, bl, orow);
  }
}

__global__ void fill_f32_kernel(float* __restrict__ p, int64_t n, float val) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) p[e] = val;
}

}  // namespace

// cu == nullptr: one sequence of N tokens; otherwise `batch` packed sequences of T
// tokens with device offsets cu[0..batch] and N = the longest length (grid.x is
// sized by it).
// Low bits of the selection key that number the blocks: enough for every block
// index of a sequence of up to N tokens.
static uint32_t block_key_mask(int64_t N, int bk) {
  const int64_t nb = (N + bk - 1) / bk;
  uint32_t m = 1;
  while ((int64_t)m < nb - 1) m = m * 2 + 1;
  return m;
}

template <int LIST, int CT, int BK>
static void launch_index_topk_ct(const uint16_t* q_idx, const uint16_t* k_idx, int64_t N, int H_kv, int k,
                                 int32_t* block_idx, const int64_t* cu, unsigned gy, int64_t T, uint32_t imask,
                                 hipStream_t stream) {
  const int64_t grid = (N * H_kv + kIdxWaves * 32 * CT - 1) / (kIdxWaves * 32 * CT);
  index_topk_kernel<LIST, CT, false, BK><<<dim3((unsigned)grid, gy), dim3(kIdxThreads), 0, stream>>>(
      q_idx, k_idx, N, H_kv, k, 0, block_idx, nullptr, cu, T, imask);
}

// Four column tiles per wave halve the staged key reads per column, but at small
// N * H_kv they leave too few workgroups: with fewer than two per CU the GPU is
// half idle (each workgroup's sweep is as long as its last query), so two tiles
// are used there instead (B_k = 64 and k > 16 always use two: four would spill).
template <int BK>
static hipError_t launch_index_topk_bk(const uint16_t* q_idx, const uint16_t* k_idx, int64_t N, int H_kv, int k,
                                       int32_t* block_idx, const int64_t* cu, int batch, int64_t T, int num_cus,
                                       hipStream_t stream) {
  const uint32_t imask = block_key_mask(N, BK);
  const unsigned gy = cu ? (unsigned)batch : 1u;
  const int64_t wg4 = (N * H_kv + kIdxWaves * 32 * 4 - 1) / (kIdxWaves * 32 * 4) * gy;
  const bool four = wg4 >= 2 * (int64_t)num_cus;
  constexpr int CT4 = BK == 128 ? 4 : 2;
  if (k <= 8) {
    if (four)
      launch_index_topk_ct<7, CT4, BK>(q_idx, k_idx, N, H_kv, k, block_idx, cu, gy, T, imask, stream);
    else
      launch_index_topk_ct<7, 2, BK>(q_idx, k_idx, N, H_kv, k, block_idx, cu, gy, T, imask, stream);
  } else if (k <= 16) {
    if (four)
      launch_index_topk_ct<15, CT4, BK>(q_idx, k_idx, N, H_kv, k, block_idx, cu, gy, T, imask, stream);
    else
      launch_index_topk_ct<15, 2, BK>(q_idx, k_idx, N, H_kv, k, block_idx, cu, gy, T, imask, stream);
  } else {
    launch_index_topk_ct<31, 2, BK>(q_idx, k_idx, N, H_kv, k, block_idx, cu, gy, T, imask, stream);
  }
  return hipGetLastError();
}

hipError_t launch_index_topk(const uint16_t* q_idx, const uint16_t* k_idx, int64_t N, int H_kv, int k,
                             int32_t* block_idx, const int64_t* cu, int batch, int64_t T, int bk, int num_cus,
                             hipStream_t stream) {
  if (bk == 64) return launch_index_topk_bk<64>(q_idx, k_idx, N, H_kv, k, block_idx, cu, batch, T, num_cus, stream);
  return launch_index_topk_bk<128>(q_idx, k_idx, N, H_kv, k, block_idx, cu, batch, T, num_cus, stream);
}

hipError_t launch_index_block_scores(const uint16_t* q_idx, const uint16_t* k_idx, int64_t N, int H_kv, int bk,
                                     float* M, hipStream_t stream) {
  const int64_t B = (N + bk - 1) / bk;
  const int64_t nM = N * H_kv * B;
  fill_f32_kernel<<<dim3(1024), dim3(256), 0, stream>>>(M, nM, -__builtin_inff());
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  constexpr int CT = 2;
  const int64_t total = N * H_kv;
  const int64_t grid = (total + kIdxWaves * 32 * CT - 1) / (kIdxWaves * 32 * CT);
  if (bk == 64)
    index_topk_kernel<1, CT, true, 64><<<dim3((unsigned)grid), dim3(kIdxThreads), 0, stream>>>(
        q_idx, k_idx, N, H_kv, 1, B, nullptr, M, nullptr, N, 0u);
  else
    index_topk_kernel<1, CT, true, 128><<<dim3((unsigned)grid), dim3(kIdxThreads), 0, stream>>>(
        q_idx, k_idx, N, H_kv, 1, B, nullptr, M, nullptr, N, 0u);
  return hipGetLastError();
}

hipError_t launch_topk_from_scores(const float* M, int64_t N, int H_kv, int64_t B, int k, int bk,
                                   int32_t* block_idx, hipStream_t stream) {
  const int64_t grid = (N * H_kv + 3) / 4;
  const int64_t chunks = (N - 1) / bk / 64 + 1;  // 64-block chunks of the longest prefix
  if (chunks > 128) return hipErrorInvalidValue;  // above the 8,192-block limit
  const dim3 g((unsigned)grid), t(256);
  if (chunks <= 16)
    topk_from_scores_kernel<16><<<g, t, 0, stream>>>(M, N, H_kv, B, k, bk, block_idx);
  else if (chunks <= 32)
    topk_from_scores_kernel<32><<<g, t, 0, stream>>>(M, N, H_kv, B, k, bk, block_idx);
  else
    topk_from_scores_long_kernel<<<g, t, 0, stream>>>(M, N, H_kv, B, k, bk, block_idx);
  return hipGetLastError();
}

}  // namespace msa
