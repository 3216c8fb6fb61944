// Main Branch kernels: inverse index, chunk list, KV-outer attention (phase 1) and
// the LSE combine (phase 2).
//
// Method: page "MiniMax Sparse Attention (MSA)" paper review, section 3, Eq. 8
// (softmax attention over the chosen blocks, shared by the G heads of a group)
// and section 5 "4.2 Sparse Attention Kernel" (KV-outer iteration with query
// gather; two-phase forward writing per-slot partials then a split-K LSE
// combine); reading notes page, section 5.4 (reverse index / query gathering,
// hot tiles pre-split into chunks with their output slots fixed in advance, so no
// atomic touches a result).
//
// Work decomposition on gfx950.  For each (group r, KV block b) the inverse index
// lists the (query, slot) pairs that chose it.  Lists are cut into fixed items of
// at most 2 * kItemChunks chunks and 512 pairs; a chunk is 128 MFMA rows = (128 / G) gathered queries x G
// heads (query concatenation).  A workgroup stages the block's K (32 KB) and V^T
// (32 KB) in LDS once per item, then for each chunk every wave computes 32 rows:
// S^T = K * Q^T and O^T = V^T * P^T on 32x32x16 bf16 MFMAs, with the softmax in
// fp32 in between.  Every pair owns its partial slot [query][group][slot], so the
// partials of hot (sink) blocks spread over many workgroups without atomics.
#include <type_traits>

#include "msa_device.h"
#include "msa_kernels.h"
#include "table_clamp.h"

namespace msa {

namespace {

// --------------------------------------------------------------------- inverse index
// Pair validity for a query at position i_rel of its sequence: 0 <= b <= b_loc =
// i_rel >> bsh (bsh = log2 B_k).  Later blocks add no token.
__device__ __forceinline__ bool pair_valid(int b, int64_t i_rel, int bsh) {
  return b >= 0 && (int64_t)b <= (i_rel >> bsh);
}

// Start of the sequence of global token i (and its index s).
__device__ __forceinline__ int64_t seq_start(const SeqInfo& si, int64_t i, int& s) {
  if (!si.cu) {
    s = 0;
    return 0;
  }
  s = si.seq_tok[i];
  return si.cu[s];
}
__device__ __forceinline__ int64_t gblock(const SeqInfo& si, int s, int b) { return si.cu ? si.bstart[s] + b : b; }

// Lists are keyed (group r, query window w, block b): list (r * nW + w) * B + b holds
// the pairs of queries in window w (WQ queries) that chose block b for group r.
// Processing lists in key order keeps the q rows being gathered (one window of one
// group) and the K/V blocks being staged (one group) small enough to stay cached.
// Blocks are numbered globally (sequence s's block b is gblock(s, b)); the blocks a
// tile of queries can choose form one range [gb_lo, gb_hi] of global blocks, which
// the LDS histogram covers.
__device__ __forceinline__ void tile_block_range(const SeqInfo& si, int64_t q0, int64_t q1, int bsh,
                                                 int64_t& gb_lo, int64_t& nh) {
  int sf, sl;
  (void)seq_start(si, q0, sf);
  const int64_t jl = seq_start(si, q1 - 1, sl);
  gb_lo = si.cu ? si.bstart[sf] : 0;
  nh = gblock(si, sl, (int)((q1 - 1 - jl) >> bsh)) - gb_lo + 1;
}

__global__ __launch_bounds__(256) void inv_count_kernel(const int32_t* __restrict__ block_idx, SeqInfo si,
                                                        int bsh, int64_t w0, int64_t W, int H_kv, int kk, int64_t B,
                                                        int TQ, int64_t WQ, int nW, int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ tcount) {
  extern __shared__ int32_t hist[];
  const int r = blockIdx.y;
  const int64_t q0 = w0 + (int64_t)blockIdx.x * TQ;
  const int64_t lbase = ((int64_t)r * nW + (q0 - w0) / WQ) * B;
  const int64_t q1 = (q0 + TQ < w0 + W) ? q0 + TQ : w0 + W;
  int64_t gb_lo, nh;
  tile_block_range(si, q0, q1, bsh, gb_lo, nh);
  for (int64_t b = threadIdx.x; b < nh; b += 256) hist[b] = 0;
  __syncthreads();
  const int64_t npairs = (q1 - q0) * kk;
  for (int64_t p = threadIdx.x; p < npairs; p += 256) {
    const int64_t i = q0 + p / kk;
    const int s = (int)(p % kk);
    int sq;
    const int64_t j0 = seq_start(si, i, sq);
    const int b = block_idx[(i * H_kv + r) * kk + s];
    if (pair_valid(b, i - j0, bsh)) atomicAdd(&hist[gblock(si, sq, b) - gb_lo], 1);
  }
  __syncthreads();
  for (int64_t b = threadIdx.x; b < nh; b += 256) {
    const int c = hist[b];
    if (c) atomicAdd(&counts[lbase + gb_lo + b], c);
    // tcount[tile][r][block]: this tile's pairs of each list (zero elsewhere).
    if (tcount) tcount[((int64_t)blockIdx.x * H_kv + r) * B + gb_lo + b] = c;
  }
}

// Exclusive scans of the per-list pair counts and item counts, in two passes over
// tiles of 1024 lists: per-tile sums, then per tile the offsets of the preceding
// tiles plus a tile-local scan, which gives the list offsets, the scatter cursors
// and the explicit item table.
constexpr int kScanTile = 1024;

// Inclusive sum over the 1024 threads of a workgroup (lds: 16 slots).
__device__ __forceinline__ int64_t block_sum_1024(int64_t x, int64_t* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m);
  __syncthreads();
  if (lane == 0) lds[wave] = x;
  __syncthreads();
  int64_t t = 0;
#pragma unroll
  for (int w = 0; w < 16; ++w) t += lds[w];
  return t;
}

// Inclusive running maximum over the 1024 threads of a workgroup (lds: 16 slots);
// *all receives the maximum over every thread.
__device__ __forceinline__ int64_t block_incl_max_1024(int64_t x, int64_t* lds, int64_t* all) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t inc = x;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int64_t y = __shfl_up(inc, m);
    if (lane >= m && y > inc) inc = y;
  }
  __syncthreads();
  if (lane == 63) lds[wave] = inc;
  __syncthreads();
  int64_t before = inc, tot = lds[0];
  for (int w = 0; w < 16; ++w) {
    const int64_t t = lds[w];
    if (w < wave && t > before) before = t;
    if (t > tot) tot = t;
  }
  *all = tot;
  return before;
}

// Exclusive scan over the 1024 threads of a workgroup (lds: 16 slots).
__device__ __forceinline__ int64_t block_excl_scan_1024(int64_t x, int64_t* lds) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int64_t inc = x;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int64_t y = __shfl_up(inc, m);
    if (lane >= m) inc += y;
  }
  __syncthreads();
  if (lane == 63) lds[wave] = inc;
  __syncthreads();
  int64_t before = 0;
  for (int w = 0; w < wave; ++w) before += lds[w];
  return before + inc - x;
}

__global__ __launch_bounds__(kScanTile) void inv_tile_sums_kernel(const int32_t* __restrict__ counts, int64_t L,
                                                                int item_q, int64_t* __restrict__ tsum) {
  __shared__ int64_t lds[16];
  const int64_t l = (int64_t)blockIdx.x * kScanTile + threadIdx.x;
  const int c = l < L ? counts[l] : 0;
  const int64_t p = block_sum_1024(c, lds);
  const int64_t it = block_sum_1024((c + item_q - 1) / item_q, lds);
  if (threadIdx.x == 0) {
    tsum[2 * blockIdx.x] = p;
    tsum[2 * blockIdx.x + 1] = it;
  }
}

__global__ __launch_bounds__(kScanTile) void inv_scan_write_kernel(const int32_t* __restrict__ counts, int64_t L,
                                                                 int64_t B, int nW, int item_q,
                                                                 const int64_t* __restrict__ tsum,
                                                                 int32_t* __restrict__ cursor,
                                                                 int4* __restrict__ items,
                                                                 int32_t* __restrict__ n_items,
                                                                 int32_t* __restrict__ lfirst,
                                                                 int32_t* __restrict__ ctr) {
  __shared__ int64_t lds[16];
  const int tile = blockIdx.x;
  if (tile == 0 && threadIdx.x < 8 * kItemCounterSets) ctr[threadIdx.x * kItemCounterStride] = 0;  // item counters
  int64_t pp = 0, ip = 0;
  for (int j = threadIdx.x; j < tile; j += kScanTile) {
    pp += tsum[2 * j];
    ip += tsum[2 * j + 1];
  }
  pp = block_sum_1024(pp, lds);
  ip = block_sum_1024(ip, lds);
  const int64_t l = (int64_t)tile * kScanTile + threadIdx.x;
  const int c = l < L ? counts[l] : 0;
  const int nit = (c + item_q - 1) / item_q;
  const int64_t poff = pp + block_excl_scan_1024(c, lds);
  const int64_t ioff = ip + block_excl_scan_1024(nit, lds);
  if (l < L) {
    cursor[l] = (int32_t)poff;
    if (lfirst) lfirst[l] = (int32_t)ioff;  // first item of list l
    for (int it = 0; it < nit; ++it) {
      const int start = (int)poff + it * item_q;
      const int cnt = (c - it * item_q < item_q) ? c - it * item_q : item_q;
      items[ioff + it] = make_int4((int)(l % B), start, cnt, (int)((l / B) / nW));
    }
  }
  if (l == L - 1) *n_items = (int32_t)(ioff + nit);
}

template <int PPT>
__global__ __launch_bounds__(256) void inv_scatter_kernel(const int32_t* __restrict__ block_idx, SeqInfo si,
                                                          int bsh, int64_t w0, int64_t W, int H_kv, int kk,
                                                          int64_t B, int TQ, int64_t WQ, int nW,
                                                          int32_t* __restrict__ cursor, int32_t* __restrict__ pairs) {
  extern __shared__ int32_t sh[];
  int32_t* hist = sh;
  int32_t* base = sh + B;
  const int r = blockIdx.y;
  const int64_t q0 = w0 + (int64_t)blockIdx.x * TQ;
  const int64_t lbase = ((int64_t)r * nW + (q0 - w0) / WQ) * B;
  const int64_t q1 = (q0 + TQ < w0 + W) ? q0 + TQ : w0 + W;
  int64_t gb_lo, nh;
  tile_block_range(si, q0, q1, bsh, gb_lo, nh);
  for (int64_t b = threadIdx.x; b < nh; b += 256) hist[b] = 0;
  __syncthreads();
  const int64_t npairs = (q1 - q0) * kk;
  int rank[PPT], slot[PPT];
#pragma unroll
  for (int u = 0; u < PPT; ++u) {
    const int64_t p = threadIdx.x + 256 * u;
    rank[u] = -1;
    slot[u] = 0;
    if (p < npairs) {
      const int64_t i = q0 + p / kk;
      const int s = (int)(p % kk);
      int sq;
      const int64_t j0 = seq_start(si, i, sq);
      const int b = block_idx[(i * H_kv + r) * kk + s];
      if (pair_valid(b, i - j0, bsh)) {
        slot[u] = (int)(gblock(si, sq, b) - gb_lo);
        rank[u] = atomicAdd(&hist[slot[u]], 1);
      }
    }
  }
  __syncthreads();
  for (int64_t b = threadIdx.x; b < nh; b += 256) {
    const int c = hist[b];
    if (c) base[b] = atomicAdd(&cursor[lbase + gb_lo + b], c);
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < PPT; ++u) {
    if (rank[u] < 0) continue;
    const int64_t p = threadIdx.x + 256 * u;
    const int64_t i = q0 + p / kk;
    const int s = (int)(p % kk);
    pairs[base[slot[u]] + rank[u]] = (int32_t)(((i - w0) << 5) | s);
  }
}

// Ordered placement (used by the backward, whose dK/dV sums follow the pair order).
// The per-tile counts become absolute bases, tile by tile in query order: list l
// of q-window wq (first tile t0) takes tiles t0 .. t1-1 in turn from its start.
__global__ __launch_bounds__(256) void inv_tile_base_kernel(int32_t* __restrict__ tcount,
                                                            const int32_t* __restrict__ cursor, int64_t B, int H_kv,
                                                            int nW, int64_t tiles, int64_t tiles_per_window) {
  const int64_t l = (int64_t)blockIdx.x * 256 + threadIdx.x;  // list (r, wq, b)
  if (l >= (int64_t)H_kv * nW * B) return;
  const int64_t b = l % B, rw = l / B;
  const int r = (int)(rw / nW), wq = (int)(rw % nW);
  const int64_t t0 = wq * tiles_per_window;
  const int64_t t1 = (t0 + tiles_per_window < tiles) ? t0 + tiles_per_window : tiles;
  int32_t run = cursor[l];  // the list's start
  for (int64_t t = t0; t < t1; ++t) {
    int32_t* c = tcount + (t * H_kv + r) * B + b;
    const int32_t n = *c;
    *c = run;
    run += n;
  }
}

// One workgroup per (query tile, group): the tile's valid pairs are sorted in LDS
// by (list, pair index) with a bitonic network, so that within each list they come
// in (query, slot) order, and written at the tile's base of each list.  A tile holds
// at most 4096 pairs (keys: list << 12 | pair index).
__global__ __launch_bounds__(256) void inv_scatter_ordered_kernel(const int32_t* __restrict__ block_idx, SeqInfo si,
                                                                  int bsh, int64_t w0, int64_t W, int H_kv, int kk,
                                                                  int64_t B, int TQ,
                                                                  const int32_t* __restrict__ tbase,
                                                                  int32_t* __restrict__ pairs) {
  constexpr int kN = 4096;
  extern __shared__ int32_t sh[];
  int32_t* keys = sh;         // kN
  int32_t* start = sh + kN;   // nh: first sorted position of each list
  __shared__ int32_t wsum[4];
  const int r = blockIdx.y;
  const int tid = threadIdx.x;
  const int64_t q0 = w0 + (int64_t)blockIdx.x * TQ;
  const int64_t q1 = (q0 + TQ < w0 + W) ? q0 + TQ : w0 + W;
  int64_t gb_lo, nh;
  tile_block_range(si, q0, q1, bsh, gb_lo, nh);
  for (int64_t b = tid; b < nh; b += 256) start[b] = 0;
  __syncthreads();
  const int npairs = (int)((q1 - q0) * kk);
  for (int p = tid; p < kN; p += 256) {
    int key = 0x7fffffff;
    if (p < npairs) {
      const int64_t i = q0 + p / kk;
      const int sl = p % kk;
      int sq;
      const int64_t j0 = seq_start(si, i, sq);
      const int b = block_idx[(i * H_kv + r) * kk + sl];
      if (pair_valid(b, i - j0, bsh)) {
        const int ls = (int)(gblock(si, sq, b) - gb_lo);
        key = (ls << 12) | p;
        atomicAdd(&start[ls], 1);  // counts only: the order of these adds is irrelevant
      }
    }
    keys[p] = key;
  }
  __syncthreads();
  // Exclusive scan of the per-list counts: thread t scans entries [t*per, (t+1)*per).
  const int per = (int)((nh + 255) / 256);
  int local = 0;
  for (int e = 0; e < per; ++e) {
    const int64_t b = (int64_t)tid * per + e;
    if (b < nh) local += start[b];
  }
  int inc = local;
  const int lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const int y = __shfl_up(inc, m);
    if (lane >= m) inc += y;
  }
  if (lane == 63) wsum[wv] = inc;
  __syncthreads();
  int before = inc - local;
  for (int w = 0; w < wv; ++w) before += wsum[w];
  for (int e = 0; e < per; ++e) {
    const int64_t b = (int64_t)tid * per + e;
    if (b < nh) {
      const int c = start[b];
      start[b] = before;
      before += c;
    }
  }
  // Bitonic sort of the kN keys, ascending.
  for (int k2 = 2; k2 <= kN; k2 <<= 1) {
    for (int j = k2 >> 1; j > 0; j >>= 1) {
      __syncthreads();
      for (int idx = tid; idx < kN; idx += 256) {
        const int partner = idx ^ j;
        if (partner > idx) {
          const int a = keys[idx], c = keys[partner];
          const bool up = (idx & k2) == 0;
          if (up ? a > c : a < c) {
            keys[idx] = c;
            keys[partner] = a;
          }
        }
      }
    }
  }
  __syncthreads();
  for (int jpos = tid; jpos < kN; jpos += 256) {
    const int key = keys[jpos];
    if (key == 0x7fffffff) continue;
    const int ls = key >> 12, p = key & 4095;
    const int64_t i = q0 + p / kk;
    const int sl = p % kk;
    const int32_t base = tbase[((int64_t)blockIdx.x * H_kv + r) * B + gb_lo + ls];
    pairs[base + (jpos - start[ls])] = (int32_t)(((i - w0) << 5) | sl);
  }
}

// --------------------------------------------------------------------- phase 1
constexpr int kAttnThreads = 256;

// The pairs of a work item live in kPairRegs<G> registers per lane: register j of
// lane l holds pair 64j + l (entries past the end repeat the last pair).  Reading
// them needs no memory access, so nothing inside the chunk loop waits on earlier
// stores.  An item holds at most 64 * kPairRegs<G> pairs.
template <int G>
constexpr int kPairRegs = G >= 4 ? 4 : 2;
// The attention kernel's items are twice as long (32 chunks, 512 pairs at G >= 4): each
// item stages its K/V block (64 KB) into LDS once, and at 128K the longer items took
// phase 1 from 12.52-12.56 to 12.31-12.35 ms (32K and B_k = 64 unchanged).
constexpr int kAttnItemMult = 2;
template <int G>
constexpr int kAttnPairRegs = kPairRegs<G> * kAttnItemMult;

// Chunk c covers the item's pairs [c*kQC, (c+1)*kQC); with G >= 4, kQC = 128/G
// divides 64, so one register holds all of them (pairs past the end are replaced
// by the last pair, which lies in the last chunk).
// (A select chain here gets turned into an indexed load from a stack copy of ip;
// a blend with an opaque uniform mask keeps ip in registers.)
template <int NR>
__device__ __forceinline__ int pick_reg(const int (&ip)[NR], int j) {
  int v = 0;
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    int m = -(int)(j == k);
    asm volatile("" : "+v"(m));
    v |= ip[k] & m;
  }
  return v;
}

// Per-lane pair index (any register): one lane shuffle per register.
template <int NR>
__device__ __forceinline__ int item_pair_v(const int (&ip)[NR], int idx) {
  int v = 0;
#pragma unroll
  for (int k = 0; k < NR; ++k) {
    const int x = __shfl(ip[k], idx & 63);
    v = (idx >> 6) == k ? x : v;
  }
  return v;
}

// Gather of one chunk's q rows, coalesced: load t of lane j fetches 16-byte chunk
// j%16 of the wave's row 4t + j/16 (16 lanes read one 256-byte head row).  Row rho
// of the wave is MFMA row wave*32 + rho = (pair cbase + (wave*32 + rho) / G, head
// (wave*32 + rho) % G); pairs past the item's end take the item's last pair (a
// valid address; see the stores for why its results may be written).  With G >= 4
// the 4 rows of a load are 4 consecutive heads of one pair, i.e. one contiguous
// 1 KB run: its base is uniform (pair read from one lane of the chunk's register
// `cur` into prs[t]) and the lane only adds lane*16 bytes.  Addresses are formed
// from the kernel's global pointer, so the loads stay global, not flat.
template <int G, int NR>
__device__ __forceinline__ void gather_q(u32x4_t (&qraw)[8], int (&prs)[8], const uint16_t* __restrict__ q,
                                         const int (&ip)[NR], int cur, int cbase, int cnt, int wave,
                                         int lane, int64_t w0, int H_q, int64_t r) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if constexpr (G >= 4) {
      const int row0 = wave * 32 + 4 * t;
      const int idx = cbase + row0 / G;
      const int pr = __builtin_amdgcn_readlane(cur, (idx < cnt ? idx : cnt - 1) & 63);
      prs[t] = pr;
      const int64_t off = ((w0 + (pr >> 5)) * H_q + r * G + row0 % G) * kDh;
      qraw[t] = *reinterpret_cast<const u32x4_t*>(q + off + lane * 8);
    } else {
      const int row = wave * 32 + 4 * t + (lane >> 4);
      const int idx = cbase + row / G;
      const int pr = item_pair_v(ip, idx < cnt ? idx : cnt - 1);
      const int64_t off = ((w0 + (pr >> 5)) * H_q + r * G + row % G) * kDh;
      qraw[t] = *reinterpret_cast<const u32x4_t*>(q + off + (lane & 15) * 8);
    }
  }
}

// BK: keys per block.  The staged tiles hold 128 keys; a 64-key block fills the
// first half, and only its two 32-key MFMA tiles (and PV steps) are computed.
template <int G, int BK>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_kvouter_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
    const int4* __restrict__ items, const int32_t* __restrict__ n_items_ptr, const int32_t* __restrict__ pairs,
    int64_t N, SeqInfo si, int H_kv, int64_t B, int nW, int kk, int64_t w0, float scale_log2,
    uint16_t* __restrict__ Opart, float2* __restrict__ Lpart, int32_t* __restrict__ ctr,
    uint64_t* __restrict__ clk) {
  constexpr int kQC = 128 / G;         // gathered queries per chunk
  constexpr int NKT = BK / 32;         // 32-key MFMA tiles per block
  __shared__ __attribute__((aligned(16))) uint8_t Ks[kBk * 256];
  __shared__ __attribute__((aligned(16))) uint8_t Vt[kDh * 256];
  __shared__ __attribute__((aligned(16))) uint8_t Ostage[4][16 * 256];  // per wave: 16 rows

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int H_q = H_kv * G;
  const int n_items = *n_items_ptr;

  // Items come from the per-XCD queues: consecutive items (mostly of one list) go
  // to the workgroups of one XCD, so the staged K/V block is read from its L2.
  // The next item is published through the first 8 bytes of wave 0's staging buffer
  // (no extra LDS: two workgroups per CU use all of it).  Thread 0 writes it after
  // wave 0's last use of that buffer for the item; every thread reads it right after
  // the item's first barrier, and the buffer is next written after the second.
  // The publishing write is waited for before the barrier explicitly: the compiler
  // emits no LDS wait ahead of the loop's first barrier, so without it another wave
  // could read the slot before the write lands.
  int64_t* const wg_item = reinterpret_cast<int64_t*>(&Ostage[0][0]);
  ItemQueue queue{ctr, n_items, (int)gridDim.x, (int)gridDim.x >> 3, (int)(blockIdx.x & 7), kItemCounterStride, 0};
  wg_clock_start(clk);
  if (tid == 0) publish_item(wg_item, queue.resolve(queue.take()));
  for (;;) {
    __syncthreads();  // the item is published; the previous item's LDS reads are done
    const int64_t item = *wg_item;
    if (item < 0) break;
    int ticket = 0;
    if (tid == 0) ticket = queue.take();  // the next item's ticket, in flight meanwhile
    const int4 it = items[item];
    const int64_t gb = it.x, r = it.w;
    const int start = it.y, cnt = it.z;
    // The list's block: block b of sequence s_item, whose tokens are [j0, j0 + seqN).
    const int s_item = si.cu ? si.seq_blk[gb] : 0;
    const int64_t b = gb - (si.cu ? si.bstart[s_item] : 0);
    const int64_t j0 = si.cu ? si.cu[s_item] : 0;
    const int64_t seqN = si.cu ? si.cu[s_item + 1] - j0 : N;

    constexpr int NR = kAttnPairRegs<G>;
    int ip[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) ip[k] = pairs[start + (64 * k + lane < cnt ? 64 * k + lane : cnt - 1)];
    {
      // Recompute the staging addresses per item rather than keeping ~40 loop-
      // invariant address registers live across the whole kernel.
      int stid = tid;
      asm volatile("" : "+v"(stid));
      const int64_t tok0 = b * BK;  // within the sequence
      const int row_stride = H_kv * kDh;
      const int nvalid = (seqN - tok0 < BK) ? (int)(seqN - tok0) : BK;
      const int64_t base = (j0 + tok0) * row_stride + r * kDh;
      stage_kv(kp + base, vp + base, row_stride, nvalid, Ks, Vt, stid);
    }
    __syncthreads();

    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int qrow = wave * 32 + l32;
    const int qs = qrow / G, g = qrow % G;
    // Chunk 0's gather; later chunks are prefetched one chunk ahead.  Gathered rows
    // are moved to the MFMA operand layout (lane l32 holds row l32) through the
    // wave's LDS buffer, 16 rows per pass, chunk c of row rho at position c ^ rho.
    uint8_t* ost = Ostage[wave];
    u32x4_t qraw[8], qop[8];
    auto to_operands = [&]() {
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int rho = 4 * tt + (lane >> 4);
          *reinterpret_cast<u32x4_t*>(ost + rho * 256 + (((lane & 15) ^ rho) << 4)) = qraw[4 * pass + tt];
        }
        if ((l32 >> 4) == pass) {
          const int rho = l32 & 15;
#pragma unroll
          for (int t = 0; t < 8; ++t)
            qop[t] = *reinterpret_cast<const u32x4_t*>(ost + rho * 256 + (((8 * h + t) ^ rho) << 4));
        }
      }
    };
    // Register holding chunk cbase's pairs (G >= 4).
    auto chunk_reg = [&](int cbase) { return pick_reg(ip, (cbase < cnt ? cbase : cnt - 1) >> 6); };
    int cur = chunk_reg(0), cur_n = cur;
    int prs[8], prs_n[8];
    gather_q<G>(qraw, prs, q, ip, cur, 0, cnt, wave_u, lane, w0, H_q, r);
    to_operands();
    for (int cb = 0; cb < cnt; cb += kQC) {
      // Keep the LDS operand reads inside the chunk loop: hoisting them (they do
      // not change across chunks) would need 256 registers per lane.
      asm volatile("" ::: "memory");
      const bool valid = cb + qs < cnt;
      int pr;  // the pair of the lane's own row
      if constexpr (G >= 4)
        pr = __shfl(cur, (valid ? cb + qs : cnt - 1) & 63);
      else
        pr = item_pair_v(ip, valid ? cb + qs : cnt - 1);
      const int64_t i_local = pr >> 5;
      const int s = pr & 31;
      const int64_t i = w0 + i_local - j0;  // query position within its sequence

      // S^T[row][qrow] with row -> key swap23(row): k-slot (h, e) of step t is dim
      // 64h + 8t + e in both operands.
      f32x16_t sacc[NKT];
      // Matrix phases run at raised wave priority, so that the other wave on the
      // SIMD fills the VALU slots with its softmax rather than competing for issue.
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        sacc[kt] = f32x16_t{};
        const int row = kt * 32 + l32;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int c = 8 * h + t;
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(Ks + row * 256 + ((c ^ (row & 15)) << 4));
          sacc[kt] = mfma_32x32x16(as_bf16x8(a), as_bf16x8(qop[t]), sacc[kt]);
        }
      }
      // Keep 8 K-operand reads in flight ahead of the MFMAs that consume them.
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int j = 0; j < 8 * NKT - 8; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);

      // Prefetch of the next chunk's q rows once the q operands are consumed: they
      // land while the softmax, PV and stores run.  (After the item's last chunk
      // this re-reads pair 0: valid addresses.)
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
      cur_n = chunk_reg(cb + kQC);
      gather_q<G>(qraw, prs_n, q, ip, cur_n, cb + kQC, cnt, wave_u, lane, w0, H_q, r);
      __builtin_amdgcn_sched_barrier(0);

      // Causal mask, only where a lane's block reaches past its query: element v of
      // tile kt is key kt*32 + 16*(v/8) + 4*((v/4)%2) + v%4 + 8h of the block.
      const int lim = (int)(i - b * BK) - 8 * h;
      if (__any(b * BK + (BK - 1) > i)) {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int off = kt * 32 + 16 * (v >> 3) + 4 * ((v >> 2) & 1) + (v & 3);
            sacc[kt][v] = off <= lim ? sacc[kt][v] : -__builtin_inff();
          }
        }
      }
      // Softmax over this block's keys in base 2 with the scale folded into one FMA.
      float mx = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[kt][v]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool empty = mx == -__builtin_inff();
      const float m2 = empty ? 0.f : mx * scale_log2;
      float l = 0.f;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[kt][v], scale_log2, -m2));
          sacc[kt][v] = p;
          l += p;
        }
      }
      l += __shfl_xor(l, 32);

      // P in bf16 as the B operand of step u: keys 32*(u/2) + 16*(u%2) + 8h + e.
      u32x4_t pb[2 * NKT];
#pragma unroll
      for (int u = 0; u < 2 * NKT; ++u) {
        const int kt = u >> 1, hf = u & 1;
        pb[u].x = pack_bf16x2(sacc[kt][8 * hf + 0], sacc[kt][8 * hf + 1]);
        pb[u].y = pack_bf16x2(sacc[kt][8 * hf + 2], sacc[kt][8 * hf + 3]);
        pb[u].z = pack_bf16x2(sacc[kt][8 * hf + 4], sacc[kt][8 * hf + 5]);
        pb[u].w = pack_bf16x2(sacc[kt][8 * hf + 6], sacc[kt][8 * hf + 7]);
      }

      // The softmax is complete before PV starts (its fp32 scores are dead), which
      // leaves registers for V^T reads in flight.
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(1);
      // Unnormalised partial (bf16) plus its base-2 max and sum for the combine.
      // The partial rows are written once and read only by the combine, so they
      // are stored non-temporally (kept from displacing the cached q and K/V).
      // Stores are unconditional: a row past the item's end computed the item's
      // last pair (same q head row, same block), so it writes that pair's partial
      // row again with the same bits (and both lane halves write their row's
      // identical (m, l)).
      const int64_t prow = ((i_local * H_kv + r) * kk + s) * G + g;
      Lpart[prow] = make_float2(empty ? -__builtin_inff() : m2, l);

      // O^T[d][qrow] = V^T[d][key] * P^T[key][qrow] in two halves of 64 dims, each
      // stored before the next starts (half the accumulators live at a time).  Lane
      // (l32, h) reads the 8-key chunk 2u + h of V^T row d = 32*dt + l32.
#pragma unroll
      for (int hd = 0; hd < 2; ++hd) {
        f32x16_t oacc[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
        for (int u = 0; u < 2 * NKT; ++u) {
          const int kc = 2 * u + h;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int d = (2 * hd + j) * 32 + l32;
            const u32x4_t va = *reinterpret_cast<const u32x4_t*>(Vt + d * 256 + ((kc ^ (d & 15)) << 4));
            oacc[j] = mfma_32x32x16(as_bf16x8(va), as_bf16x8(pb[u]), oacc[j]);
          }
        }
        // V^T-operand reads run 8 ahead of their MFMAs.
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 1);
#pragma unroll
        for (int j = 0; j < 4 * NKT - 8; ++j) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 1);
        if (hd == 1) {
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_setprio(0);
        }

        // The half tile leaves the MFMA with lane (l32, h) holding dims 32j + 8c +
        // 4h .. +3 (c = 0..3) of row l32.  Through the wave's LDS buffer (half-row
        // rho at rho*128, 16-byte chunk x at position x ^ (rho & 7)) it is
        // re-read as 8 half-rows of 128 bytes per instruction.
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            u32x2_t pk;
            pk.x = pack_bf16x2(oacc[j][4 * c + 0], oacc[j][4 * c + 1]);
            pk.y = pack_bf16x2(oacc[j][4 * c + 2], oacc[j][4 * c + 3]);
            *reinterpret_cast<u32x2_t*>(ost + l32 * 128 + (((4 * j + c) ^ (l32 & 7)) << 4) + 8 * h) = pk;
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int rho = 8 * u + (lane >> 3), ch = lane & 7;
          const u32x4_t val = *reinterpret_cast<const u32x4_t*>(ost + rho * 128 + ((ch ^ (rho & 7)) << 4));
          if constexpr (G >= 8) {
            // Half-rows 8u..8u+7 are heads g0..g0+7 of the pair of gather load 2u:
            // uniform base.
            const int row0 = wave_u * 32 + 8 * u;
            const int pu = prs[2 * u];
            const int64_t prow0 = (((int64_t)(pu >> 5) * H_kv + r) * kk + (pu & 31)) * G + row0 % G;
            __builtin_nontemporal_store(
                val, reinterpret_cast<u32x4_t*>(Opart + prow0 * kDh + 64 * hd + (lane >> 3) * kDh + ch * 8));
          } else if constexpr (G == 4) {
            // Half-rows 8u..8u+3 and 8u+4..8u+7 belong to the pairs of gather loads
            // 2u and 2u+1.
            const int row = wave_u * 32 + rho;
            // A blend with an opaque mask: a plain select by lane half becomes an
            // indexed load from a stack copy of prs.
            int hm = -(lane >> 5);
            asm volatile("" : "+v"(hm));
            const int pu = (prs[2 * u + 1] & hm) | (prs[2 * u] & ~hm);
            const int64_t prow_s = (((int64_t)(pu >> 5) * H_kv + r) * kk + (pu & 31)) * G + row % G;
            __builtin_nontemporal_store(val, reinterpret_cast<u32x4_t*>(Opart + prow_s * kDh + 64 * hd + ch * 8));
          } else {
            const int row = wave * 32 + rho;
            const int pu = item_pair_v(ip, cb + row / G < cnt ? cb + row / G : cnt - 1);
            const int64_t prow_s = (((int64_t)(pu >> 5) * H_kv + r) * kk + (pu & 31)) * G + row % G;
            __builtin_nontemporal_store(val, reinterpret_cast<u32x4_t*>(Opart + prow_s * kDh + 64 * hd + ch * 8));
          }
        }
      }
      // The next chunk's q rows to the operand layout here, after this chunk's
      // stores, so that the wait for them counts those stores as still in flight.
      to_operands();
      cur = cur_n;
#pragma unroll
      for (int t = 0; t < 8; ++t) prs[t] = prs_n[t];

    }
    if (tid == 0) publish_item(wg_item, queue.resolve(ticket));  // read by all after the next barrier
  }
  wg_clock_end(clk);
}

// --------------------------------------------------------------------- phase 2
// LSE merge of the valid slots' normalised partials.  One wave per (query, group,
// run of GW heads): lane -> (head, run of 2*GW dims); all slots' loads are issued
// before any arithmetic so that a wave keeps 16 x (4*GW) bytes per lane in flight.
// SEQ: packed sequences (si.cu set).  A compile-time switch, since a run-time branch
// on si.cu here changes the scheduling of the partial loads below (measured: 147
// instead of 95 VGPRs at G = 8 and a 10% slower combine).
template <int G, int KMAX, bool SEQ>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ Opart,
                                                      const float2* __restrict__ Lpart,
                                                      const int32_t* __restrict__ block_idx, SeqInfo si,
                                                      int bsh, int64_t w0, int64_t W, int H_kv, int kk,
                                                      float* __restrict__ o, float* __restrict__ lse) {
  constexpr int GW = G < 32 ? G : 32;       // heads per wave
  constexpr int LPH = 64 / GW;               // lanes per head
  constexpr int DPL = kDh / LPH;             // dims per lane (2*GW)
  constexpr int HPW = G / GW;                // waves per (query, group)
  // Consecutive waves take consecutive (query, group) rows, so the workgroups in
  // flight stream one contiguous region of partials and of o.
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (gw >= W * H_kv * HPW) return;
  const int hw = (int)(gw % HPW);
  const int64_t ir = gw / HPW;               // (i_local, r); ir < 2^32 (W <= 2^20, H_kv < 2^12)
  const int64_t i_local = (uint32_t)ir / (uint32_t)H_kv;
  const int r = (int)((uint32_t)ir - (uint32_t)i_local * (uint32_t)H_kv);
  const int64_t i = w0 + i_local;
  const int64_t i_rel = SEQ ? i - si.cu[si.seq_tok[i]] : i;
  const int g = hw * GW + lane / LPH;
  const int d0 = (lane % LPH) * DPL;
  const int H_q = H_kv * G;
  const int32_t* sel = block_idx + (i * H_kv + r) * kk;
  const int64_t pbase = ir * kk;             // partial row of slot 0 (times G)

  // Slot s: unnormalised partial o_s with base-2 max m_s and sum l_s;
  // o = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s, lse = (M + log2 L) ln 2.
  // Slot validity is the same for the whole wave.  Invalid slots re-read the first
  // valid slot's row with weight 0, so every slot's load can be in flight at once.
  bool valid[KMAX];
  int first = -1;
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    valid[s] = s < kk && pair_valid(sel[s < kk ? s : 0], i_rel, bsh);
    if (valid[s] && first < 0) first = s;
  }
  float* orow = o + (i * H_q + r * G + g) * kDh + d0;
  if (first < 0) {
#pragma unroll
    for (int d = 0; d < DPL; ++d) orow[d] = 0.f;
    if (lane % LPH == 0) lse[i * H_q + r * G + g] = -__builtin_inff();
    return;
  }
  // Above 16 slots the (m, l) pairs are read twice (for the maximum, then per slot)
  // rather than held: holding 32 of them took the kernel from 5 to 3 waves per SIMD.
  constexpr bool kHold = KMAX <= 16;
  constexpr int NH = kHold ? KMAX : 1;
  float ms[NH], ls[NH];
  float mstar = -__builtin_inff();
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    const float2 ml = Lpart[(pbase + (valid[s] ? s : first)) * G + g];
    const float m = valid[s] ? ml.x : -__builtin_inff();
    if constexpr (kHold) {
      ms[s] = m;
      ls[s] = ml.y;
    }
    mstar = fmaxf(mstar, m);
  }
  float acc[DPL];
#pragma unroll
  for (int d = 0; d < DPL; ++d) acc[d] = 0.f;
  float L = 0.f;
#pragma unroll
  for (int s = 0; s < KMAX; ++s) {
    float m_s, l_s;
    if constexpr (kHold) {
      m_s = ms[s];
      l_s = ls[s];
    } else {
      const float2 ml = Lpart[(pbase + (valid[s] ? s : first)) * G + g];
      m_s = valid[s] ? ml.x : -__builtin_inff();
      l_s = ml.y;
    }
    const float wgt = valid[s] ? __builtin_amdgcn_exp2f(m_s - mstar) : 0.f;
    L += wgt * l_s;
    const uint16_t* src = Opart + ((pbase + (valid[s] ? s : first)) * G + g) * kDh + d0;
    // DPL bf16 values = DPL/2 dwords, read with the widest aligned vector.
    uint32_t w[DPL / 2];
    if constexpr (DPL >= 8) {
#pragma unroll
      for (int d = 0; d < DPL; d += 8) {
        const uint4 u = *reinterpret_cast<const uint4*>(src + d);
        w[d / 2] = u.x;
        w[d / 2 + 1] = u.y;
        w[d / 2 + 2] = u.z;
        w[d / 2 + 3] = u.w;
      }
    } else if constexpr (DPL == 4) {
      const uint2 u = *reinterpret_cast<const uint2*>(src);
      w[0] = u.x;
      w[1] = u.y;
    } else {
      w[0] = *reinterpret_cast<const uint32_t*>(src);
    }
#pragma unroll
    for (int m = 0; m < DPL / 2; ++m) {
      acc[2 * m] += wgt * __uint_as_float(w[m] << 16);
      acc[2 * m + 1] += wgt * __uint_as_float(w[m] & 0xffff0000u);
    }
  }
  const float invL = 1.f / L;
  if constexpr (DPL >= 4) {
#pragma unroll
    for (int d = 0; d < DPL; d += 4)
      *reinterpret_cast<float4*>(orow + d) =
          make_float4(acc[d] * invL, acc[d + 1] * invL, acc[d + 2] * invL, acc[d + 3] * invL);
  } else {
    *reinterpret_cast<float2*>(orow) = make_float2(acc[0] * invL, acc[1] * invL);
  }
  if (lane % LPH == 0) lse[i * H_q + r * G + g] = (mstar + __log2f(L)) * kLn2;
}

// Tables of a varlen call (one workgroup).  First the caller's offsets cu_in[0..batch]
// are copied to cu as sanitized_offset() of their running maximum: 0, non-decreasing,
// T at the end, so the sequences partition [0, T) even if the table is malformed (a
// well-formed table is copied unchanged).  Then, from that copy, bstart[s] = the sum
// over earlier sequences of their block counts ceil(len / B_k), bstart[batch] = the
// total.
__global__ __launch_bounds__(kScanTile) void seq_block_starts_kernel(const int64_t* __restrict__ cu_in, int batch,
                                                                   int64_t T, int bk, int64_t* __restrict__ cu,
                                                                   int32_t* __restrict__ bstart) {
  __shared__ int64_t lds[16];
  int64_t pmax = INT64_MIN;
  for (int s0 = 0; s0 <= batch; s0 += kScanTile) {
    const int s = s0 + threadIdx.x;
    int64_t tile_max;
    const int64_t run = block_incl_max_1024(s <= batch ? cu_in[s] : INT64_MIN, lds, &tile_max);
    if (s <= batch) cu[s] = sanitized_offset(run > pmax ? run : pmax, s, batch, T);
    if (tile_max > pmax) pmax = tile_max;
  }
  __syncthreads();  // the copy is read back below by other threads of the workgroup
  int64_t carry = 0;
  for (int s0 = 0; s0 < batch; s0 += kScanTile) {
    const int s = s0 + threadIdx.x;
    const int64_t nb = s < batch ? (cu[s + 1] - cu[s] + bk - 1) / bk : 0;
    const int64_t ex = block_excl_scan_1024(nb, lds);
    if (s < batch) bstart[s] = (int32_t)(carry + ex);
    carry += block_sum_1024(nb, lds);
  }
  if (threadIdx.x == 0) bstart[batch] = (int32_t)carry;
}

// One workgroup per sequence: the sequence of each of its tokens and blocks.
__global__ __launch_bounds__(256) void seq_fill_kernel(const int64_t* __restrict__ cu,
                                                       const int32_t* __restrict__ bstart,
                                                       int32_t* __restrict__ seq_tok, int32_t* __restrict__ seq_blk) {
  const int s = blockIdx.x;
  for (int64_t t = cu[s] + threadIdx.x; t < cu[s + 1]; t += 256) seq_tok[t] = s;
  for (int64_t gb = bstart[s] + threadIdx.x; gb < bstart[s + 1]; gb += 256) seq_blk[gb] = s;
}

// --------------------------------------------------------------------- KL alignment
// Eq. 9-10 on the selected token set, KV-outer like phase 1 (same lists, items,
// gather and K staging).  Per pair (query i, group r, slot s, block b), over the
// block's tokens j <= i:
//   Z = sum_j P_j,  A = sum_j P_j ln P_j,  C = sum_j P_j S_j,
//   m = max_j S_j,  l = sum_j exp(S_j - m),
// with S_j = <q_idx[i][r], k_idx[j]> / sqrt(d_idx) the index score and
// P_j = (1/G) sum_h exp(s_hj - lse_h) the teacher: the mean of the group's head
// softmaxes, each normalised by its head's final log partition lse_h from the main
// pass.  Summed over the slots, KL(P || P_idx) = A - C + Z * LSE_idx with
// LSE_idx = ln sum_s l_s e^{m_s}.  Z is 1 up to rounding; it is kept exact.

// K_idx block -> LDS in the staged K tile's key order: row rho (128 B = 8 chunks of
// 16 B) holds key swap23(rho), chunk c at position c ^ ((rho >> 1) & 7).
__device__ __forceinline__ void stage_kidx(const uint16_t* __restrict__ kib, int nvalid, uint8_t* KIs, int tid) {
  const int c = tid & 7;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int rho = (tid >> 3) + 32 * m;
    const int key = swap23(rho);
    const int kr = key < nvalid ? key : nvalid - 1;
    u32x4_t val = *reinterpret_cast<const u32x4_t*>(kib + kr * kDidx + c * 8);
    if (key >= nvalid) val = u32x4_t{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4_t*>(KIs + rho * 128 + ((c ^ ((rho >> 1) & 7)) << 4)) = val;
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

// Sum / max over the 32 lanes of a wave half (every lane gets the result).
__device__ __forceinline__ float half_sum(float x) {
  x += dpp_f<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_f<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_f<0x141>(x);  // row_half_mirror
  x += dpp_f<0x140>(x);  // row_mirror
  return x + __shfl_xor(x, 16);
}
__device__ __forceinline__ float half_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  x = fmaxf(x, dpp_f<0x141>(x));
  x = fmaxf(x, dpp_f<0x140>(x));
  return fmaxf(x, __shfl_xor(x, 16));
}

// Score tiles here are Q K^T (q rows as MFMA rows): element v of lane (l32, h) is q
// row 8*(v/4) + 4h + v%4 of the wave's 32 (query slot x head) and column l32, key
// kt*32 + swap23(l32) of the block.  A query's heads then sit in GL consecutive
// elements of one lane (and, for G >= 8, in both lane halves), so the teacher's
// head mean is a few in-lane adds, and the per-query terms are computed NQ times
// per lane instead of once per head.
template <int G>
struct KlRows {
  static constexpr int GL = G <= 4 ? G : G / 2;  // heads of one query per lane
  static constexpr int NQ = 16 / GL;             // queries per lane and tile
  static constexpr bool kCross = G >= 8;         // the other heads are in lane ^ 32
};

// Register budget of kl_pair_kernel<G, BK>.  A lane keeps the running sums of its
// KlRows<G>::NQ queries (16 at G = 1) and the next chunk's operands in flight, which
// leaves the compiler little slack at two workgroups per CU.  Per variant, chosen
// from the compiler's resource-usage report so that none spills registers:
//  - G <= 2 runs one workgroup per CU (its running sums do not fit the 256
//    registers of two);
//  - G = 4 and G = 16, and G = 8 with 128-key blocks when it keeps the index log
//    partition (not GIVEN), walk their key tiles in a loop rather than unrolled
//    (the unrolled form spills at two workgroups per CU);
//  - the key tiles are walked by two copies of the loop, with and without the
//    causal mask (only a query's own block needs it), except for G = 4 with
//    128-key blocks and not GIVEN, which spills with both copies.
template <int G, int BK, bool GIVEN>
struct KlRegs {
  static constexpr int kBlocksPerCU = G <= 2 ? 1 : 2;
  static constexpr int kTileUnroll = (G == 4 || G == 16 || (G == 8 && !GIVEN && BK == 128)) ? 1 : BK / 32;
  static constexpr bool kSplitMask = !(G == 4 && BK == 128 && !GIVEN);
};

// Index score scale 1 / sqrt(d_idx), in natural and base-2 units.
constexpr float kIdxScale = 0.125f;
constexpr float kIdxScaleLog2 = kIdxScale * kLog2e;
static_assert(kDidx == 64, "kIdxScale is 1 / sqrt(64)");

// BK: keys per block (64 or 128); a 64-key block fills the first half of the
// staged tiles, and only its two 32-key tiles are computed.  GIVEN: LSE_idx is an
// input (from msa_sparse_attn_fwd_lse_idx), so the index log partition is not
// accumulated and a pair's partial is (A, C, Z) alone.
template <int G, int BK, bool GIVEN>
__global__ __launch_bounds__(kAttnThreads, (KlRegs<G, BK, GIVEN>::kBlocksPerCU)) void kl_pair_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kp, const uint16_t* __restrict__ q_idx,
    const uint16_t* __restrict__ k_idx, const float* __restrict__ lse, const int4* __restrict__ items,
    const int32_t* __restrict__ n_items_ptr, const int32_t* __restrict__ pairs, int64_t N, int H_kv, int64_t B,
    int nW, int kk, int64_t w0, float scale_log2, float* __restrict__ part, int32_t* __restrict__ ctr) {
  constexpr int kQC = 128 / G;
  constexpr int GL = KlRows<G>::GL, NQ = KlRows<G>::NQ;
  static_assert(G <= 32, "a query's heads must lie in one wave");
  static_assert((G & (G - 1)) == 0, "G is a power of two");
  constexpr float kLog2G = (float)__builtin_ctz(G);
  __shared__ __attribute__((aligned(16))) uint8_t Ks[kBk * 256];
  __shared__ __attribute__((aligned(16))) uint8_t KIs[kBk * 128];
  __shared__ __attribute__((aligned(16))) uint8_t Qs[4][32 * 256];  // per wave: its 32 q rows

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int H_q = H_kv * G;
  const int n_items = *n_items_ptr;
  // Items from the per-XCD queues, as in the attention kernel; the next item is
  // published through the first 8 bytes of wave 0's q rows, which are next written
  // after the item's second barrier.
  int64_t* const wg_item = reinterpret_cast<int64_t*>(&Qs[0][0]);
  ItemQueue queue{ctr, n_items, (int)gridDim.x, (int)gridDim.x >> 3, (int)(blockIdx.x & 7), kItemCounterStride, 0};
  if (tid == 0) publish_item(wg_item, queue.resolve(queue.take()));
  for (;;) {
    __syncthreads();  // the item is published; the previous item's LDS reads are done
    const int64_t item = *wg_item;
    if (item < 0) break;
    int ticket = 0;
    if (tid == 0) ticket = queue.take();  // the next item's ticket, in flight meanwhile
    const int4 it = items[item];
    const int64_t b = it.x, r = it.w;
    const int start = it.y, cnt = it.z;

    constexpr int NR = kPairRegs<G>;
    int ip[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) ip[k] = pairs[start + (64 * k + lane < cnt ? 64 * k + lane : cnt - 1)];
    {
      int stid = tid;
      asm volatile("" : "+v"(stid));
      const int64_t tok0 = b * BK;
      const int nvalid = (N - tok0 < BK) ? (int)(N - tok0) : BK;
      stage_k(kp + tok0 * H_kv * kDh + r * kDh, H_kv * kDh, nvalid, Ks, stid);
      stage_kidx(k_idx + tok0 * kDidx, nvalid, KIs, stid);
    }
    __syncthreads();

    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int qrow = wave * 32 + l32;  // the lane's own row (operand side)
    const int qs = qrow / G, g = qrow % G;
    uint8_t* qs_w = Qs[wave];
    u32x4_t qraw[8];
    // The chunk's gathered q rows wait in the wave's LDS rows (row rho, 16-byte
    // chunk c at position c ^ (rho & 15)) and are read as MFMA operands tile by
    // tile (the block's K, K_idx and these rows fill the 80 KB that two
    // workgroups per CU allow).
    auto to_lds = [&]() {
      int ln = lane;  // addresses formed per call, not held across the loop
      asm volatile("" : "+v"(ln));
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int rho = 4 * t + (ln >> 4);
        *reinterpret_cast<u32x4_t*>(qs_w + rho * 256 + (((ln & 15) ^ (rho & 15)) << 4)) = qraw[t];
      }
    };
    auto chunk_reg = [&](int cbase) { return pick_reg(ip, (cbase < cnt ? cbase : cnt - 1) >> 6); };
    // The pair of the lane's own row in chunk cbase (rows past the item's end take
    // its last pair).
    auto lane_pair = [&](int cbase, int curv) {
      const int idx = cbase + qs < cnt ? cbase + qs : cnt - 1;
      if constexpr (G >= 4)
        return __shfl(curv, idx & 63);
      else
        return item_pair_v(ip, idx);
    };
    // Index query of the lane's own row (dims 32h + 8t .. +7 for step t) and its
    // head's main log partition in base 2.
    auto lane_operands = [&](int prv, u32x4_t (&qi)[4], float& l2) {
      int hh = h;  // opaque: the lane's base address is formed per call, not held
      asm volatile("" : "+v"(hh));
      const int64_t iq = w0 + (prv >> 5);
      const uint16_t* src = q_idx + (iq * H_kv + r) * kDidx + 32 * hh;
#pragma unroll
      for (int t = 0; t < 4; ++t) qi[t] = *reinterpret_cast<const u32x4_t*>(src + 8 * t);
      l2 = fmaf(lse[iq * H_q + r * G + g], kLog2e, kLog2G);  // log2(G): the head mean's 1/G
    };

    int cur = chunk_reg(0), cur_n = cur;
    int prs[8];
    gather_q<G>(qraw, prs, q, ip, cur, 0, cnt, wave_u, lane, w0, H_q, r);
    int pr = lane_pair(0, cur);
    u32x4_t qi_op[4];
    float l2own;
    lane_operands(pr, qi_op, l2own);
    to_lds();
    for (int cb = 0; cb < cnt; cb += kQC) {
      asm volatile("" ::: "memory");
      // Output rows of this lane (row 8*(v/4) + 4h + v%4 is the own row of lane
      // with that l32): lse of all 16, pair of each query.
      // (The source lanes are formed from an opaque base each chunk: as constants
      // they would be hoisted and hold 16 + NQ registers across the loop.)
      float l2v[16];
      int prq[NQ];
      int hb = 4 * h;
      asm volatile("" : "+v"(hb));
#pragma unroll
      for (int v = 0; v < 16; ++v) l2v[v] = __shfl(l2own, 8 * (v >> 2) + hb + (v & 3));
#pragma unroll
      for (int qq = 0; qq < NQ; ++qq) {
        const int v0 = qq * GL;
        prq[qq] = __shfl(pr, 8 * (v0 >> 2) + hb + (v0 & 3));
      }

      // Next chunk's q rows and per-lane operands, in flight during this chunk.
      cur_n = chunk_reg(cb + kQC);
      gather_q<G>(qraw, prs, q, ip, cur_n, cb + kQC, cnt, wave_u, lane, w0, H_q, r);
      const int pr_n = lane_pair(cb + kQC, cur_n);
      u32x4_t qi_n[4];
      float l2_n;
      lane_operands(pr_n, qi_n, l2_n);

      int ln = l32;
      asm volatile("" : "+v"(ln));
      const uint8_t* ks_row = Ks + ln * 256;
      const uint8_t* ki_row = KIs + ln * 128;
      const uint8_t* q_row = qs_w + ln * 256;
      const int ks_sw = ln & 15, ki_sw = (ln >> 1) & 7;
      const int koff0 = swap23(ln);  // key of column l32 in tile 0
      int lim[NQ];
      bool part_blk = false;
#pragma unroll
      for (int qq = 0; qq < NQ; ++qq) {
        lim[qq] = (int)(w0 + (prq[qq] >> 5) - b * BK);
        part_blk |= lim[qq] < BK - 1;
      }
      part_blk = __any(part_blk);
      // Running sums per query over the lane's keys, in the units that cost no
      // instruction per key: R = <q_idx, k_idx> unscaled (S = R / sqrt(d_idx)), and
      // base-2 logarithms; the constant factors are applied once per block below.
      //   Z = sum P,  C = sum P R,  A = sum P log2 P,
      //   l = sum 2^((R - mx) c), mx = max R, c = log2(e) / sqrt(d_idx).
      // P log2 P uses max(P, FLT_MIN) in the logarithm, so P = 0 adds 0 without a
      // select.  l takes one exponential per key: 2^(-|R - mx| c) either scales the
      // old sum (R above the running max) or is the key's own term.
      float A[NQ], C[NQ], Z[NQ], mx[NQ], l[NQ];
#pragma unroll
      for (int qq = 0; qq < NQ; ++qq) {
        A[qq] = C[qq] = Z[qq] = l[qq] = 0.f;
        mx[qq] = -__builtin_inff();
      }
      auto tile = [&](int kt, auto masked) {
        constexpr bool MASKED = decltype(masked)::value;
        f32x16_t sacc = f32x16_t{}, iacc = f32x16_t{};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int c = 8 * h + t;
          const u32x4_t aq = *reinterpret_cast<const u32x4_t*>(q_row + ((c ^ ks_sw) << 4));
          const u32x4_t bk = *reinterpret_cast<const u32x4_t*>(ks_row + kt * 32 * 256 + ((c ^ ks_sw) << 4));
          sacc = mfma_32x32x16(as_bf16x8(aq), as_bf16x8(bk), sacc);
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int c = 4 * h + t;
          const u32x4_t bk = *reinterpret_cast<const u32x4_t*>(ki_row + kt * 32 * 128 + ((c ^ ki_sw) << 4));
          iacc = mfma_32x32x16(as_bf16x8(qi_op[t]), as_bf16x8(bk), iacc);
        }
        const int koff = kt * 32 + koff0;
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq) {
          // Teacher P: the mean over the group's heads (1/G is in l2v).
          float ps = __builtin_amdgcn_exp2f(fmaf(sacc[qq * GL], scale_log2, -l2v[qq * GL]));
#pragma unroll
          for (int e = 1; e < GL; ++e) {
            const int v = qq * GL + e;
            ps += __builtin_amdgcn_exp2f(fmaf(sacc[v], scale_log2, -l2v[v]));
          }
          if constexpr (KlRows<G>::kCross) ps += __shfl_xor(ps, 32);
          const bool in = !MASKED || koff <= lim[qq];
          const float P = in ? ps : 0.f;
          const float R = iacc[qq * GL];
          Z[qq] += P;
          C[qq] = fmaf(P, R, C[qq]);
          A[qq] = fmaf(P, __log2f(fmaxf(P, __FLT_MIN__)), A[qq]);
          if constexpr (!GIVEN) {
            const float d = in ? R - mx[qq] : -__builtin_inff();
            const float ex = __builtin_amdgcn_exp2f(-fabsf(d) * kIdxScaleLog2);
            const bool up = d > 0.f;
            l[qq] = up ? fmaf(l[qq], ex, 1.f) : l[qq] + ex;
            mx[qq] = up ? R : mx[qq];
          }
        }
      };
      if (!KlRegs<G, BK, GIVEN>::kSplitMask || part_blk) {
#pragma unroll KlRegs<G, BK, GIVEN>::kTileUnroll
        for (int kt = 0; kt < BK / 32; ++kt) tile(kt, std::true_type{});
      } else {
#pragma unroll KlRegs<G, BK, GIVEN>::kTileUnroll
        for (int kt = 0; kt < BK / 32; ++kt) tile(kt, std::false_type{});
      }
      // Sum over the block's keys (the 32 columns of a lane half, 4 tiles each).
#pragma unroll
      for (int qq = 0; qq < NQ; ++qq) {
        const float a = half_sum(A[qq]) * kLn2, c = half_sum(C[qq]) * kIdxScale, z = half_sum(Z[qq]);
        float M = 0.f, ls = 0.f;
        if constexpr (!GIVEN) {
          const float Mr = half_max(mx[qq]);
          const float ref = Mr == -__builtin_inff() ? 0.f : Mr;
          ls = half_sum(l[qq] * __builtin_amdgcn_exp2f((mx[qq] - ref) * kIdxScaleLog2));
          M = Mr * kIdxScale;
        }
        const bool writer = l32 == 0 && (!KlRows<G>::kCross || h == 0);
        if (writer) {
          const int pq = prq[qq];
          float* dst = part + (((int64_t)(pq >> 5) * H_kv + r) * kk + (pq & 31)) * kKlPart;
          *reinterpret_cast<float4*>(dst) = make_float4(a, c, z, M);
          if constexpr (!GIVEN) dst[4] = ls;
        }
      }

      to_lds();
      cur = cur_n;
      pr = pr_n;
      l2own = l2_n;
#pragma unroll
      for (int t = 0; t < 4; ++t) qi_op[t] = qi_n[t];
    }
    if (tid == 0) publish_item(wg_item, queue.resolve(ticket));  // read by all after the next barrier
  }
}

// Per (query, group): sum of the valid slots' partials, then KL and LSE_idx (lse_in
// set: LSE_idx is given, and only KL is written).
__global__ __launch_bounds__(256) void kl_combine_kernel(const float* __restrict__ part,
                                                         const int32_t* __restrict__ block_idx, int64_t w0,
                                                         int64_t W, int H_kv, int kk, int bsh,
                                                         const float* __restrict__ lse_in,
                                                         float* __restrict__ kl, float* __restrict__ lse_idx) {
  const int64_t ir = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (ir >= W * H_kv) return;
  const int64_t i = w0 + ir / H_kv;
  const int32_t* sel = block_idx + (w0 * H_kv + ir) * kk;
  float A = 0.f, C = 0.f, Z = 0.f, M = -__builtin_inff(), L = 0.f;
  for (int s = 0; s < kk; ++s) {
    if (!pair_valid(sel[s], i, bsh)) continue;
    const float* src = part + (ir * kk + s) * kKlPart;
    const float4 a = *reinterpret_cast<const float4*>(src);
    const float l = src[4];
    A += a.x;
    C += a.y;
    Z += a.z;
    if (lse_in || a.w == -__builtin_inff()) continue;
    if (a.w > M) {
      L = L * __expf(M - a.w) + l;
      M = a.w;
    } else {
      L += l * __expf(a.w - M);
    }
  }
  const int64_t o = w0 * H_kv + ir;
  if (lse_in) {
    const float lse_i = lse_in[o];
    kl[o] = lse_i == -__builtin_inff() ? 0.f : A - C + lse_i * Z;
  } else if (M == -__builtin_inff()) {
    kl[o] = 0.f;
    lse_idx[o] = -__builtin_inff();
  } else {
    const float lse_i = M + __logf(L);
    kl[o] = A - C + lse_i * Z;
    lse_idx[o] = lse_i;
  }
}

// Fixed-order reduction of kl[0..n): workgroup w sums its contiguous share in fp64.
__global__ __launch_bounds__(256) void kl_sum_kernel(const float* __restrict__ kl, int64_t n,
                                                     double* __restrict__ partial) {
  __shared__ double red[256];
  const int64_t share = (n + gridDim.x - 1) / gridDim.x;
  const int64_t e0 = (int64_t)blockIdx.x * share;
  const int64_t e1 = e0 + share < n ? e0 + share : n;
  double acc = 0.0;
  for (int64_t e = e0 + threadIdx.x; e < e1; e += 256) acc += (double)kl[e];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) partial[blockIdx.x] = red[0];
}

__global__ __launch_bounds__(256) void kl_mean_kernel(const double* __restrict__ partial, int np, int64_t n,
                                                      float* __restrict__ loss) {
  __shared__ double red[256];
  red[threadIdx.x] = (int)threadIdx.x < np ? partial[threadIdx.x] : 0.0;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = (float)(red[0] / (double)n);
}

// --------------------------------------------------------------------- LSE_idx
// The index distribution's log partition over the selected tokens (Eq. 9's P^idx
// normaliser), emitted with the forward as the pages' main pass emits it (paper
// review, section 5, 4.3): LSE_idx[i][r] = ln sum over the tokens j <= i of the
// row's selected blocks of exp(S_j), S_j = <q_idx[i][r], k_idx[j]> / sqrt(d_idx).
// It walks the main pass's lists (items of one (group, block)), so each index-key
// block is staged once per list; per (query, group, slot) pair it writes the
// block's base-2 max and sum, and lse_idx_combine_kernel merges a row's slots.
//
// Per item: the block's index keys go to LDS in the staged key order (stage_kidx);
// the pairs are taken 128 at a time, wave w's lanes l32 owning pair 32w + l32 (both
// lane halves).  S^T = K_idx . q_idx^T on 32x32x16 MFMAs puts 16 keys of the pair
// in each lane (element v of tile kt is key kt*32 + 16(v/8) + 4((v/4)%2) + v%4 + 8h,
// as in phase 1), so the max and the sum over keys are in-lane, then across the
// two lane halves.  The q_idx row of the pair is the B operand (k-slot (h, e) of
// step t is dim 32h + 8t + e, matching chunk 4h + t of the staged key rows).
template <int BK>
__global__ __launch_bounds__(256) void lse_idx_pair_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_idx, const int4* __restrict__ items,
    const int32_t* __restrict__ n_items_ptr, const int32_t* __restrict__ pairs, int64_t N, SeqInfo si, int H_kv,
    int kk, int64_t w0, float2* __restrict__ lidx, int32_t* __restrict__ ctr) {
  constexpr int NKT = BK / 32;
  constexpr float kScale2 = kIdxScaleLog2;
  __shared__ __attribute__((aligned(16))) uint8_t KIs[kBk * 128];
  __shared__ int64_t wg_item;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int n_items = *n_items_ptr;
  ItemQueue queue{ctr, n_items, (int)gridDim.x, (int)gridDim.x >> 3, (int)(blockIdx.x & 7), kItemCounterStride, 0};
  if (tid == 0) publish_item(&wg_item, queue.resolve(queue.take()));
  for (;;) {
    __syncthreads();  // the item is published; the previous item's LDS reads are done
    const int64_t item = wg_item;
    if (item < 0) break;
    int ticket = 0;
    if (tid == 0) ticket = queue.take();
    const int4 it = items[item];
    const int64_t gb = it.x, r = it.w;
    const int start = it.y, cnt = it.z;
    const int s_item = si.cu ? si.seq_blk[gb] : 0;
    const int64_t b = gb - (si.cu ? si.bstart[s_item] : 0);
    const int64_t j0 = si.cu ? si.cu[s_item] : 0;
    const int64_t seqN = si.cu ? si.cu[s_item + 1] - j0 : N;
    const int64_t tok0 = b * BK;
    const int nvalid = (seqN - tok0 < BK) ? (int)(seqN - tok0) : BK;
    stage_kidx(k_idx + (j0 + tok0) * kDidx, nvalid, KIs, tid);
    __syncthreads();

    const uint8_t* ki_row = KIs + l32 * 128;
    const int ki_sw = (l32 >> 1) & 7;
    for (int p0 = 0; p0 < cnt; p0 += 128) {
      const int pi = p0 + wave * 32 + l32;
      const int pr = pairs[start + (pi < cnt ? pi : cnt - 1)];
      const int64_t i_local = pr >> 5;
      const int64_t i = w0 + i_local;  // global row
      const uint16_t* src = q_idx + (i * H_kv + r) * kDidx + 32 * h;
      u32x4_t qb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) qb[t] = *reinterpret_cast<const u32x4_t*>(src + 8 * t);
      // Causal limit of this lane's keys: key kt*32 + off + 8h is visible iff off <= lim.
      const int lim = (int)(i - j0 - tok0) - 8 * h;
      float m = -__builtin_inff(), l = 0.f;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        f32x16_t acc = f32x16_t{};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const u32x4_t a = *reinterpret_cast<const u32x4_t*>(ki_row + kt * 32 * 128 + (((4 * h + t) ^ ki_sw) << 4));
          acc = mfma_32x32x16(as_bf16x8(a), as_bf16x8(qb[t]), acc);
        }
        float sv[16];
        float tm = -__builtin_inff();
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int off = kt * 32 + 16 * (v >> 3) + 4 * ((v >> 2) & 1) + (v & 3);
          sv[v] = off <= lim ? acc[v] * kScale2 : -__builtin_inff();
          tm = fmaxf(tm, sv[v]);
        }
        const float nm = fmaxf(m, tm);
        if (nm != -__builtin_inff()) {
          float add = 0.f;
#pragma unroll
          for (int v = 0; v < 16; ++v) add += __builtin_amdgcn_exp2f(sv[v] - nm);
          l = l * __builtin_amdgcn_exp2f(m - nm) + add;
          m = nm;
        }
      }
      // The other lane half holds the pair's other keys.
      const float mo = __shfl_xor(m, 32), lo = __shfl_xor(l, 32);
      const float M = fmaxf(m, mo);
      const float L = (m == -__builtin_inff() ? 0.f : l * __builtin_amdgcn_exp2f(m - M)) +
                      (mo == -__builtin_inff() ? 0.f : lo * __builtin_amdgcn_exp2f(mo - M));
      if (h == 0 && pi < cnt) lidx[(i_local * H_kv + r) * kk + (pr & 31)] = make_float2(M, L);
    }
    if (tid == 0) publish_item(&wg_item, queue.resolve(ticket));
  }
}

// LSE_idx[i][r] from the row's valid slots (same validity rule as the combine):
// ln of sum_s 2^m_s l_s; -inf when no slot is valid.  One thread per (query, group).
__global__ __launch_bounds__(256) void lse_idx_combine_kernel(const float2* __restrict__ lidx,
                                                              const int32_t* __restrict__ block_idx, SeqInfo si,
                                                              int bsh, int64_t w0, int64_t W, int H_kv, int kk,
                                                              float* __restrict__ lse_idx) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (i_local, r)
  if (t >= W * H_kv) return;
  const int64_t i = w0 + t / H_kv;
  int s_seq;
  const int64_t i_rel = i - seq_start(si, i, s_seq);
  const int32_t* sel = block_idx + (i * H_kv + t % H_kv) * kk;
  float M = -__builtin_inff(), L = 0.f;
  for (int s = 0; s < kk; ++s) {
    if (!pair_valid(sel[s], i_rel, bsh)) continue;
    const float2 ml = lidx[t * kk + s];
    if (ml.x == -__builtin_inff()) continue;
    if (ml.x > M) {
      L = L * __builtin_amdgcn_exp2f(M - ml.x) + ml.y;
      M = ml.x;
    } else {
      L += ml.y * __builtin_amdgcn_exp2f(ml.x - M);
    }
  }
  lse_idx[i * H_kv + t % H_kv] = M == -__builtin_inff() ? -__builtin_inff() : (M + __log2f(L)) * kLn2;
}

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t val) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) p[e] = val;
}

}  // namespace

// Query tile of the inverse-index passes: a power of two with at most 4096 pairs.
static int inv_tile_queries(int kk) {
  int tq = 1;
  while (tq * 2 * kk <= 4096) tq *= 2;
  return tq;
}

SeqTables seq_tables_layout(int64_t T, int batch, int64_t Bt) {
  SeqTables S{};
  if (batch <= 0) return S;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  S.cu = take(sizeof(int64_t) * ((size_t)batch + 1));
  S.bstart = take(sizeof(int32_t) * ((size_t)batch + 1));
  S.seq_tok = take(sizeof(int32_t) * (size_t)T);
  S.seq_blk = take(sizeof(int32_t) * (size_t)Bt);
  S.total = off;
  return S;
}

hipError_t launch_seq_tables(const int64_t* cu_in, int batch, int64_t T, int bk, uint8_t* ws, const SeqTables& S,
                             hipStream_t stream) {
  int32_t* bstart = reinterpret_cast<int32_t*>(ws + S.bstart);
  int64_t* cu = reinterpret_cast<int64_t*>(ws + S.cu);
  seq_block_starts_kernel<<<dim3(1), dim3(kScanTile), 0, stream>>>(cu_in, batch, T, bk, cu, bstart);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  seq_fill_kernel<<<dim3((unsigned)batch), dim3(256), 0, stream>>>(cu, bstart, reinterpret_cast<int32_t*>(ws + S.seq_tok),
                                                                   reinterpret_cast<int32_t*>(ws + S.seq_blk));
  return hipGetLastError();
}

AttnWorkspace attn_workspace_layout(int64_t W, int H_q, int H_kv, int kk, int64_t B, int parts) {
  AttnWorkspace L{};
  // q-locality window of 64*B queries (a multiple of 4096, so every inverse-index
  // tile lies in one window): each K/V block is staged once per (group, window)
  // list, so fewer, longer lists cut the staging traffic; measured at 128K, 64*B
  // (two windows) beat 8*B (16 windows) by 6% and equals a single window.
  int64_t WQ = ((64 * B + 4095) / 4096) * 4096;
  if (WQ > W) WQ = ((W + 4095) / 4096) * 4096;
  L.WQ = WQ;
  L.nW = (int)((W + WQ - 1) / WQ);
  const int64_t lists = (int64_t)H_kv * L.nW * B;
  const int64_t max_pairs = W * H_kv * kk;
  const int G = H_q / H_kv;
  // The attention and KL kernels keep an item's pairs in registers: at most 256
  // pairs for G >= 4 and 128 otherwise, twice that for the attention.
  const int mult = parts == kPartsAttn ? kAttnItemMult : 1;
  const int max_q = (G >= 4 ? 256 : 128) * mult;
  const int chunks = kItemChunks * mult;
  const int item_fwd = chunks * (128 / G) < max_q ? chunks * (128 / G) : max_q;
  const int item_q = parts == kPartsBwd ? kBwdItemPairs : item_fwd;
  const int64_t max_items = (max_pairs + item_q - 1) / item_q + lists;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  L.counts = take(sizeof(int32_t) * lists);
  L.tsum = take(sizeof(int64_t) * 2 * ((lists + kScanTile - 1) / kScanTile));
  L.cursor = take(sizeof(int32_t) * lists);
  L.n_items = take(sizeof(int32_t) * 4);
  L.ctr = take(sizeof(int32_t) * kItemCounterStride * 8 * kItemCounterSets);
  L.items = take(sizeof(int4) * max_items);
  L.pairs = take(sizeof(int32_t) * max_pairs);
  if (parts == kPartsKl) {
    L.opart = take(sizeof(float) * kKlPart * max_pairs);
    L.lpart = take(0);
  } else if (parts == kPartsBwd) {
    L.opart = take(sizeof(uint16_t) * (max_pairs * G + 1) * kDh);  // bf16 dQ row per (pair, head), + a dummy row
    L.lpart = take(sizeof(float) * max_items * 2 * kBk * kDh);   // dK and dV block per item
  } else {
    L.opart = take(sizeof(uint16_t) * max_pairs * G * kDh);
    L.lpart = take(sizeof(float2) * max_pairs * G);
  }
  L.lidx = take(parts == kPartsAttn ? sizeof(float2) * max_pairs : 0);  // LSE_idx per pair
  L.lfirst = take(parts == kPartsBwd ? sizeof(int32_t) * lists : 0);
  // Per-tile list counts (then bases) of the ordered placement: tiles x H_kv x B.
  const int64_t tq = inv_tile_queries(kk);
  L.tcount = take(parts == kPartsBwd ? sizeof(int32_t) * ((W + tq - 1) / tq) * H_kv * B : 0);
  L.total = off;
  L.max_items = max_items;
  L.item_q = item_q;
  return L;
}

// Inverse index of one query window: per-list pair counts, their scan into list
// offsets and the item table, then the scatter of the (query, slot) pairs.
hipError_t launch_inverse_index(const int32_t* block_idx, int64_t B, const SeqInfo& si, int bsh, int H_kv, int kk,
                                int64_t w0, int64_t W, uint8_t* ws, const AttnWorkspace& L, hipStream_t stream,
                                int32_t* lfirst, bool ordered) {
  const int64_t lists = (int64_t)H_kv * L.nW * B;
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* cursor = reinterpret_cast<int32_t*>(ws + L.cursor);
  int32_t* n_items = reinterpret_cast<int32_t*>(ws + L.n_items);
  int4* items = reinterpret_cast<int4*>(ws + L.items);
  int32_t* pairs = reinterpret_cast<int32_t*>(ws + L.pairs);
  hipError_t e;
  fill_i32_kernel<<<dim3(256), dim3(256), 0, stream>>>(counts, lists, 0);
  e = hipGetLastError();
  if (e != hipSuccess) return e;

  // Query tiles of the inverse-index passes hold at most 4096 pairs (16 per thread).
  const int TQ = inv_tile_queries(kk);
  const int64_t qtiles = (W + TQ - 1) / TQ;
  const dim3 igrid((unsigned)qtiles, (unsigned)H_kv);
  const size_t lds_count = sizeof(int32_t) * B;
  int32_t* tcount = ordered ? reinterpret_cast<int32_t*>(ws + L.tcount) : nullptr;
  if (ordered) {
    fill_i32_kernel<<<dim3(256), dim3(256), 0, stream>>>(tcount, qtiles * H_kv * B, 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  inv_count_kernel<<<igrid, dim3(256), lds_count, stream>>>(block_idx, si, bsh, w0, W, H_kv, kk, B, TQ, L.WQ,
                                                             L.nW, counts, tcount);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const unsigned tiles = (unsigned)((lists + kScanTile - 1) / kScanTile);
  int64_t* tsum = reinterpret_cast<int64_t*>(ws + L.tsum);
  inv_tile_sums_kernel<<<dim3(tiles), dim3(kScanTile), 0, stream>>>(counts, lists, L.item_q, tsum);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  inv_scan_write_kernel<<<dim3(tiles), dim3(kScanTile), 0, stream>>>(counts, lists, B, L.nW, L.item_q, tsum, cursor,
                                                                    items, n_items, lfirst,
                                                                    reinterpret_cast<int32_t*>(ws + L.ctr));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ordered) {
    inv_tile_base_kernel<<<dim3((unsigned)((lists + 255) / 256)), dim3(256), 0, stream>>>(
        tcount, cursor, B, H_kv, L.nW, qtiles, L.WQ / TQ);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    inv_scatter_ordered_kernel<<<igrid, dim3(256), sizeof(int32_t) * 4096 + lds_count, stream>>>(
        block_idx, si, bsh, w0, W, H_kv, kk, B, TQ, tcount, pairs);
    return hipGetLastError();
  }
  inv_scatter_kernel<16><<<igrid, dim3(256), 2 * lds_count, stream>>>(block_idx, si, bsh, w0, W, H_kv, kk, B,
                                                                      TQ, L.WQ, L.nW, cursor, pairs);
  return hipGetLastError();
}

hipError_t launch_sparse_attn_window(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const int32_t* block_idx, int64_t N, int64_t B, const SeqInfo& si, int bk,
                                     int H_q, int H_kv, int kk, float scale, int64_t w0, int64_t W, int num_cus,
                                     float* o, float* lse, uint8_t* ws, const AttnWorkspace& L, hipStream_t stream,
                                     const hipEvent_t* events, uint64_t* clk, const uint16_t* q_idx,
                                     const uint16_t* k_idx, float* lse_idx) {
  const int bsh = bk == 64 ? 6 : 7;
  const int G = H_q / H_kv;
  const int32_t* n_items = reinterpret_cast<const int32_t*>(ws + L.n_items);
  const int4* items = reinterpret_cast<const int4*>(ws + L.items);
  const int32_t* pairs = reinterpret_cast<const int32_t*>(ws + L.pairs);
  uint16_t* opart = reinterpret_cast<uint16_t*>(ws + L.opart);
  float2* lpart = reinterpret_cast<float2*>(ws + L.lpart);

  hipError_t e;
  if (events && (e = hipEventRecord(events[0], stream)) != hipSuccess) return e;
  if ((e = launch_inverse_index(block_idx, B, si, bsh, H_kv, kk, w0, W, ws, L, stream)) != hipSuccess) return e;

  int64_t grid = (int64_t)num_cus * 2;
  if (grid > L.max_items) grid = L.max_items;
  grid = ((grid + 7) / 8) * 8;
  const float scale_log2 = scale * kLog2e;
  int32_t* ctr = reinterpret_cast<int32_t*>(ws + L.ctr);
  if (events && (e = hipEventRecord(events[1], stream)) != hipSuccess) return e;
  switch (G) {
#define MSA_ATTN_CASE(GG)                                                                            \
  case GG:                                                                                           \
    if (bk == 64)                                                                                    \
      attn_kvouter_kernel<GG, 64><<<dim3((unsigned)grid), dim3(kAttnThreads), 0, stream>>>(          \
          q, k, v, items, n_items, pairs, N, si, H_kv, B, L.nW, kk, w0, scale_log2, opart, lpart, ctr, clk);\
    else                                                                                             \
      attn_kvouter_kernel<GG, 128><<<dim3((unsigned)grid), dim3(kAttnThreads), 0, stream>>>(         \
          q, k, v, items, n_items, pairs, N, si, H_kv, B, L.nW, kk, w0, scale_log2, opart, lpart, ctr, clk);\
    break;
    MSA_ATTN_CASE(1)
    MSA_ATTN_CASE(2)
    MSA_ATTN_CASE(4)
    MSA_ATTN_CASE(8)
    MSA_ATTN_CASE(16)
    MSA_ATTN_CASE(32)
    MSA_ATTN_CASE(64)
    MSA_ATTN_CASE(128)
#undef MSA_ATTN_CASE
    default:
      return hipErrorInvalidValue;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;

  if (events && (e = hipEventRecord(events[2], stream)) != hipSuccess) return e;
  const int64_t waves = W * H_kv * (G > 32 ? G / 32 : 1);
  const dim3 cgrid((unsigned)((waves + 3) / 4));
  switch (G) {
#define MSA_COMBINE_CASE(GG)                                                                          \
  case GG:                                                                                           \
    if (kk <= 16 && !si.cu)                                                                          \
      combine_kernel<GG, 16, false><<<cgrid, dim3(256), 0, stream>>>(opart, lpart, block_idx, si, bsh, w0, W, H_kv, kk, o, \
                                                                     lse);                           \
    else if (kk <= 16)                                                                               \
      combine_kernel<GG, 16, true><<<cgrid, dim3(256), 0, stream>>>(opart, lpart, block_idx, si, bsh, w0, W, H_kv, kk, o, \
                                                                    lse);                            \
    else if (!si.cu)                                                                                 \
      combine_kernel<GG, 32, false><<<cgrid, dim3(256), 0, stream>>>(opart, lpart, block_idx, si, bsh, w0, W, H_kv, kk, o, \
                                                                     lse);                           \
    else                                                                                             \
      combine_kernel<GG, 32, true><<<cgrid, dim3(256), 0, stream>>>(opart, lpart, block_idx, si, bsh, w0, W, H_kv, kk, o, \
                                                                    lse);                            \
    break;
    MSA_COMBINE_CASE(1)
    MSA_COMBINE_CASE(2)
    MSA_COMBINE_CASE(4)
    MSA_COMBINE_CASE(8)
    MSA_COMBINE_CASE(16)
    MSA_COMBINE_CASE(32)
    MSA_COMBINE_CASE(64)
    MSA_COMBINE_CASE(128)
#undef MSA_COMBINE_CASE
    default:
      return hipErrorInvalidValue;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (events && (e = hipEventRecord(events[3], stream)) != hipSuccess) return e;
  if (!lse_idx) return hipSuccess;
  // LSE_idx over the same lists (after the events, so that the phase times above
  // stay those of the plain forward).
  float2* lidx = reinterpret_cast<float2*>(ws + L.lidx);
  int32_t* ctr1 = ctr + 8 * kItemCounterStride;  // the second counter set
  int64_t lgrid = (int64_t)num_cus * 4;
  if (lgrid > L.max_items) lgrid = L.max_items;
  lgrid = ((lgrid + 7) / 8) * 8;
  if (bk == 64)
    lse_idx_pair_kernel<64><<<dim3((unsigned)lgrid), dim3(256), 0, stream>>>(q_idx, k_idx, items, n_items, pairs, N,
                                                                             si, H_kv, kk, w0, lidx, ctr1);
  else
    lse_idx_pair_kernel<128><<<dim3((unsigned)lgrid), dim3(256), 0, stream>>>(q_idx, k_idx, items, n_items, pairs, N,
                                                                              si, H_kv, kk, w0, lidx, ctr1);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  lse_idx_combine_kernel<<<dim3((unsigned)((W * H_kv + 255) / 256)), dim3(256), 0, stream>>>(
      lidx, block_idx, si, bsh, w0, W, H_kv, kk, lse_idx);
  return hipGetLastError();
}

hipError_t launch_sparse_kl_window(const uint16_t* q, const uint16_t* k, const uint16_t* q_idx,
                                   const uint16_t* k_idx, const float* lse, const int32_t* block_idx, int64_t N,
                                   int64_t B, int bk, int H_q, int H_kv, int kk, float scale, int64_t w0, int64_t W,
                                   int num_cus, const float* lse_idx_in, float* kl, float* lse_idx, uint8_t* ws,
                                   const AttnWorkspace& L, hipStream_t stream) {
  const int G = H_q / H_kv;
  const int bsh = bk == 64 ? 6 : 7;
  hipError_t e = launch_inverse_index(block_idx, B, SeqInfo{}, bsh, H_kv, kk, w0, W, ws, L, stream);
  if (e != hipSuccess) return e;
  const int32_t* n_items = reinterpret_cast<const int32_t*>(ws + L.n_items);
  const int4* items = reinterpret_cast<const int4*>(ws + L.items);
  const int32_t* pairs = reinterpret_cast<const int32_t*>(ws + L.pairs);
  float* part = reinterpret_cast<float*>(ws + L.opart);
  int32_t* ctr = reinterpret_cast<int32_t*>(ws + L.ctr);
  int64_t grid = (int64_t)num_cus * 2;
  if (grid > L.max_items) grid = L.max_items;
  grid = ((grid + 7) / 8) * 8;
  const float scale_log2 = scale * kLog2e;
  switch (G) {
#define MSA_KL_LAUNCH(GG, BB, GV)                                                                          \
  kl_pair_kernel<GG, BB, GV><<<dim3((unsigned)grid), dim3(kAttnThreads), 0, stream>>>(                     \
      q, k, q_idx, k_idx, lse, items, n_items, pairs, N, H_kv, B, L.nW, kk, w0, scale_log2, part, ctr)
#define MSA_KL_CASE(GG)                                                                                    \
  case GG:                                                                                                 \
    if (bk == 64 && lse_idx_in)                                                                            \
      MSA_KL_LAUNCH(GG, 64, true);                                                                         \
    else if (bk == 64)                                                                                     \
      MSA_KL_LAUNCH(GG, 64, false);                                                                        \
    else if (lse_idx_in)                                                                                   \
      MSA_KL_LAUNCH(GG, 128, true);                                                                        \
    else                                                                                                   \
      MSA_KL_LAUNCH(GG, 128, false);                                                                       \
    break;
    MSA_KL_CASE(1)
    MSA_KL_CASE(2)
    MSA_KL_CASE(4)
    MSA_KL_CASE(8)
    MSA_KL_CASE(16)
    MSA_KL_CASE(32)
#undef MSA_KL_CASE
#undef MSA_KL_LAUNCH
    default:
      return hipErrorInvalidValue;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t rows = W * H_kv;
  kl_combine_kernel<<<dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream>>>(
      part, block_idx, w0, W, H_kv, kk, bsh, lse_idx_in, kl, lse_idx);
  return hipGetLastError();
}

hipError_t launch_kl_loss(const float* kl, int64_t n, double* partial, float* loss, hipStream_t stream) {
  kl_sum_kernel<<<dim3(kKlLossParts), dim3(256), 0, stream>>>(kl, n, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  kl_mean_kernel<<<dim3(1), dim3(256), 0, stream>>>(partial, kKlLossParts, n, loss);
  return hipGetLastError();
}

}  // namespace msa
