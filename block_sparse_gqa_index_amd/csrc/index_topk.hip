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

namespace msa {

namespace {

constexpr int kIdxWaves = 8;
constexpr int kIdxThreads = kIdxWaves * kWave;
constexpr int kIdxLoads = kBk * 8 / kIdxThreads;  // 16-byte chunks of a staged block per thread
constexpr int kIdxBlocksPerCU = 8 / kIdxWaves;     // two waves per SIMD

// Stage key block b of k_idx into LDS: 128 rows x 8 chunks of 16 B, chunk c of row
// j stored at chunk position c ^ ((j >> 1) & 7): the 16 rows a 16-lane LDS pass
// reads then fall on 16 different 16-byte bank groups.
__device__ __forceinline__ void idx_load_block(const uint16_t* __restrict__ k_idx, int64_t N,
                                               int64_t b, int tid, uint4 (&r)[kIdxLoads]) {
#pragma unroll
  for (int m = 0; m < kIdxLoads; ++m) {
    const int cidx = tid + kIdxThreads * m;
    const int key = cidx >> 3, c = cidx & 7;
    const int64_t j = b * kBk + key;
    r[m] = j < N ? *reinterpret_cast<const uint4*>(k_idx + j * kDidx + c * 8) : make_uint4(0, 0, 0, 0);
  }
}

__device__ __forceinline__ void idx_store_block(uint8_t* buf, int tid, const uint4 (&r)[kIdxLoads]) {
#pragma unroll
  for (int m = 0; m < kIdxLoads; ++m) {
    const int cidx = tid + kIdxThreads * m;
    const int key = cidx >> 3, c = cidx & 7;
    *reinterpret_cast<uint4*>(buf + key * 128 + ((c ^ ((key >> 1) & 7)) << 4)) = r[m];
  }
}

// Block maxima of one staged key block for the lane's CT column tiles (raw dot
// products; the 1/sqrt(d_idx) scale is applied by the caller when needed).
// The 4 x CT output tiles are software-pipelined over two accumulators: the four
// MFMAs of tile j+1 are issued before tile j is max-reduced, so the VALU reduction
// of one tile runs under the matrix work of the next.
template <int CT>
__device__ __forceinline__ void idx_tile_reduce(const f32x16_t& acc, int64_t qi, int64_t b, int kt, bool need_mask,
                                                int h, float& bmax) {
  if (need_mask) {
    // key b*128 + kt*32 + 8*(v/4) + 4h + v%4 is visible iff its offset <= lim
    int64_t lim64 = qi - (b * kBk + kt * 32 + 4 * h);
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
// belongs to block kt / (4 / NS) of the staged tile.
template <int CT, int NS>
__device__ __forceinline__ void idx_block_max(const uint8_t* buf, const uint4 (&qop)[CT][4], const int64_t (&qi)[CT],
                                              int64_t b, bool need_mask, int h, int l32, float (&bmax)[CT][NS]) {
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
      idx_tile_reduce<CT>(acc[pj & 1], qi[pct], b, pkt, need_mask, h, bmax[pct][pkt / kPerBlock]);
    }
  }
  {
    constexpr int pj = kTiles - 1, pkt = pj / CT, pct = pj % CT;
    idx_tile_reduce<CT>(acc[pj & 1], qi[pct], b, pkt, need_mask, h, bmax[pct][pkt / kPerBlock]);
  }
  __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
    for (int u = 0; u < NS; ++u) bmax[ct][u] = fmaxf(bmax[ct][u], __shfl_xor(bmax[ct][u], 32));
  }
}

// LIST: register list length (>= k-1); CT: 32-column tiles per wave.
// WRITE_M: emit block scores M[c][b] (scaled) instead of selecting.
//
// Selection: staged tiles are swept in pairs (b, b+1).  After the pair, both lane
// halves hold every block maximum of their column; the lower half offers tile b's
// blocks to its list and the upper half tile b+1's to its own, so one insertion
// sequence serves two tiles.  The two lists (blocks of even / odd tiles) are
// merged at the end.
// Sequences: with cu == nullptr the call is one sequence of N tokens; otherwise
// cu[0..batch] (device) are the packed sequence offsets, grid.y is the sequence and
// grid.x the column tile within it (tiles past the sequence's end exit).  Every
// position below (queries, blocks, keys) is relative to the sequence start j0;
// columns and output rows are global.
template <int LIST, int CT, bool WRITE_M, int BK>
__global__ __launch_bounds__(kIdxThreads, kIdxBlocksPerCU) void index_topk_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx_all, int64_t N_all, int H_kv,
    int k, int64_t B, int32_t* __restrict__ block_idx, float* __restrict__ M, const int64_t* __restrict__ cu) {
  constexpr int NS = kBk / BK;  // blocks per staged 128-key tile
  constexpr int kColsPerWave = 32 * CT;
  constexpr int kCols = kIdxWaves * kColsPerWave;
  constexpr int kBlkBytes = kBk * kDidx * 2;
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][2][kBlkBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t j0 = cu ? cu[blockIdx.y] : 0;
  const int64_t N = cu ? cu[blockIdx.y + 1] - j0 : N_all;  // tokens of this sequence
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

  int64_t col[CT], qi[CT];
  uint4 qop[CT][4];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    col[ct] = gcol0 + wave_c0 + ct * 32 + l32;
    const bool ok = wave_c0 + ct * 32 + l32 < total;
    qi[ct] = ok ? (wave_c0 + ct * 32 + l32) / H_kv : -1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      qop[ct][ks] = ok ? *reinterpret_cast<const uint4*>(q_idx + col[ct] * kDidx + ks * 16 + 8 * h)
                       : make_uint4(0, 0, 0, 0);
  }

  TopList<LIST> list[CT];
  if constexpr (!WRITE_M) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) list[ct].init();
  }

  uint4 pre[2][kIdxLoads];
  idx_load_block(k_idx, N, 0, tid, pre[0]);
  if (b_last >= 1) idx_load_block(k_idx, N, 1, tid, pre[1]);
  int step = 0;
  for (int64_t b = 0; b <= b_last; b += 2, ++step) {
    const bool two = b + 1 <= b_last;
    uint8_t* buf0 = kbuf[step & 1][0];
    uint8_t* buf1 = kbuf[step & 1][1];
    idx_store_block(buf0, tid, pre[0]);
    if (two) idx_store_block(buf1, tid, pre[1]);
    __syncthreads();
    if (b + 2 <= b_last) idx_load_block(k_idx, N, b + 2, tid, pre[0]);
    if (b + 3 <= b_last) idx_load_block(k_idx, N, b + 3, tid, pre[1]);

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
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        // block (b + h) * NS + u: this lane half's tile
        const int64_t blk = (b + h) * NS + u;
        const float x = h ? m1[ct][u] : m0[ct][u];
        if constexpr (WRITE_M) {
          if (qi[ct] >= 0 && (h == 0 || two) && blk < B) M[col[ct] * B + blk] = x * 0.125f;  // 1/sqrt(64), exact
        } else {
          // Blocks before the local one compete; the local block is forced later.
          if (blk < qi[ct] / BK) list[ct].offer(x, (int)blk);
        }
      }
    }
  }

  if constexpr (!WRITE_M) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      // Merge the even-block list (lower half) with the odd-block list (upper half):
      // own run descending, partner's run reversed, one bitonic merge.
      uint64_t key[2 * (LIST + 1)];
#pragma unroll
      for (int j = 0; j < LIST; ++j) {
        const uint64_t mine = rank_key(list[ct].v[j], list[ct].b[j]);
        const float ov = __shfl_xor(list[ct].v[j], 32);
        const int ob = __shfl_xor(list[ct].b[j], 32);
        key[j] = mine;
        key[2 * (LIST + 1) - 1 - j] = rank_key(ov, ob);
      }
      key[LIST] = 0ull;
      key[LIST + 1] = 0ull;
      bitonic_merge_desc<2 * (LIST + 1)>(key);
      if (qi[ct] < 0) continue;
      // Lanes l and l+32 now hold identical merged runs; each writes half of the row.
      int cand[LIST + 1];
#pragma unroll
      for (int j = 0; j < LIST; ++j) {
        const int blk = rank_key_block(key[j]);
        cand[j] = (j < k - 1 && blk >= 0) ? blk : 0x7fffffff;
      }
      cand[LIST] = 0x7fffffff;
      int32_t out[LIST + 1];
      write_selection<LIST + 1>(cand, k, (int)(qi[ct] / BK), out);
      int32_t* row = block_idx + col[ct] * k;
      const int half = (k + 1) >> 1;
#pragma unroll
      for (int t = 0; t <= LIST; ++t) {
        if (t < k && ((t < half) == (h == 0))) row[t] = out[t];
      }
    }
  }
}

// Top-k of given block scores (the split form of the selection), one wave per
// (query, group) row, four rows per workgroup.  Block b < b_loc of the row has the
// 64-bit key rank_key(score, b): score first, then the lower block.  The k-1 best
// keys are found without sorting the row:
//  1. lane l takes blocks l, l + 64, ... (coalesced across the wave; all of the
//     row's R chunks of 64 stay in registers) and keeps its best key.  The (k-1)-th best of
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
  if (kk == 0) {
    if (lane == 0) orow[0] = bl;
    return;
  }
  if (bl <= kk) {  // every causal block is chosen
    for (int t = lane; t < k; t += 64) orow[t] = t <= bl ? t : -1;
    return;
  }
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
  // t0: the lane best that exactly kk-1 lane bests exceed (nonzero keys are distinct
  // and at least kk+1 lanes hold one).
  s_lbest[w][lane] = lbest;
  wave_lds_sync();
  int above = 0;
#pragma unroll 8
  for (int l = 0; l < 64; ++l) above += s_lbest[w][l] > lbest;
  const uint64_t who = __ballot(above == kk - 1);
  const int wl = __builtin_ctzll(who);
  const uint64_t t0 = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(lbest >> 32), wl) << 32) |
                      (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)lbest, wl);

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
    // 3. Keep the candidates that fewer than kk others beat, in block order.
    int S = 0;
    for (int m0 = 0; m0 < C; m0 += 64) {
      const int ci = m0 + lane;
      const uint64_t key = ci < C ? s_cand[w][ci] : ~0ull;
      int beat = 0;
      for (int cj = 0; cj < C; ++cj) beat += s_cand[w][cj] > key;
      const bool keep = ci < C && beat < kk;
      const uint64_t bal = __ballot(keep);
      if (keep) orow[S + lane_prefix(bal)] = rank_key_block(key);
      S += __popcll(bal);
    }
    if (lane == 0) orow[S] = bl;  // S == kk
  } else {
    // kk rounds of wave arg-max, each below the previous round's key; lane t keeps
    // round t's block, then the kk blocks are placed by their rank.
    uint64_t prev = ~0ull;
    int mine = 0x7fffffff;
    for (int t = 0; t < kk; ++t) {
      uint64_t best = 0;
#pragma unroll
      for (int j = 0; j < R; ++j) {
        if (j < nch) {
          const int b = j * 64 + lane;
          const uint64_t key = b < bl ? rank_key(x[j], b) : 0ull;
          best = (key < prev && key > best) ? key : best;
        }
      }
      prev = wave_max_u64(best);
      if (lane == t) mine = rank_key_block(prev);
    }
    wave_lds_sync();
    s_cand[w][lane] = (uint64_t)(uint32_t)mine;
    wave_lds_sync();
    if (lane < kk) {
      int pos = 0;
      for (int t = 0; t < kk; ++t) pos += (int)s_cand[w][t] < mine;
      orow[pos] = mine;
    }
    if (lane == 0) orow[kk] = bl;
  }
}

__global__ void fill_f32_kernel(float* __restrict__ p, int64_t n, float val) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) p[e] = val;
}

}  // namespace

// cu == nullptr: one sequence of N tokens; otherwise `batch` packed sequences with
// device offsets cu[0..batch] and N = the longest length (grid.x is sized by it).
template <int BK>
static hipError_t launch_index_topk_bk(const uint16_t* q_idx, const uint16_t* k_idx, int64_t N, int H_kv, int k,
                                       int32_t* block_idx, const int64_t* cu, int batch, hipStream_t stream) {
  const int64_t total = N * H_kv;
  const unsigned gy = cu ? (unsigned)batch : 1u;
  if (k <= 8) {
    constexpr int CT = 2;
    const int64_t grid = (total + kIdxWaves * 32 * CT - 1) / (kIdxWaves * 32 * CT);
    index_topk_kernel<7, CT, false, BK><<<dim3((unsigned)grid, gy), dim3(kIdxThreads), 0, stream>>>(
        q_idx, k_idx, N, H_kv, k, 0, block_idx, nullptr, cu);
  } else if (k <= 16) {
    constexpr int CT = 2;
    const int64_t grid = (total + kIdxWaves * 32 * CT - 1) / (kIdxWaves * 32 * CT);
    index_topk_kernel<15, CT, false, BK><<<dim3((unsigned)grid, gy), dim3(kIdxThreads), 0, stream>>>(
        q_idx, k_idx, N, H_kv, k, 0, block_idx, nullptr, cu);
  } else {
    constexpr int CT = 1;
    const int64_t grid = (total + kIdxWaves * 32 * CT - 1) / (kIdxWaves * 32 * CT);
    index_topk_kernel<31, CT, false, BK><<<dim3((unsigned)grid, gy), dim3(kIdxThreads), 0, stream>>>(
        q_idx, k_idx, N, H_kv, k, 0, block_idx, nullptr, cu);
  }
  return hipGetLastError();
}

hipError_t launch_index_topk(const uint16_t* q_idx, const uint16_t* k_idx, int64_t N, int H_kv, int k,
                             int32_t* block_idx, const int64_t* cu, int batch, int bk, hipStream_t stream) {
  if (bk == 64) return launch_index_topk_bk<64>(q_idx, k_idx, N, H_kv, k, block_idx, cu, batch, stream);
  return launch_index_topk_bk<128>(q_idx, k_idx, N, H_kv, k, block_idx, cu, batch, stream);
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
        q_idx, k_idx, N, H_kv, 1, B, nullptr, M, nullptr);
  else
    index_topk_kernel<1, CT, true, 128><<<dim3((unsigned)grid), dim3(kIdxThreads), 0, stream>>>(
        q_idx, k_idx, N, H_kv, 1, B, nullptr, M, nullptr);
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
  else if (chunks <= 64)
    topk_from_scores_kernel<64><<<g, t, 0, stream>>>(M, N, H_kv, B, k, bk, block_idx);
  else
    topk_from_scores_kernel<128><<<g, t, 0, stream>>>(M, N, H_kv, B, k, bk, block_idx);
  return hipGetLastError();
}

}  // namespace msa
