// Main Branch backward: the gradients of Eq. 8 with respect to q, k and v for a
// fixed selection (the selection itself has no gradient).
//
// Method: page "MiniMax Sparse Attention (MSA)" paper review, section 3, Eq. 8
// (softmax attention over the chosen blocks) differentiated; reading notes page,
// section 5.4 (the backward walks the same KV-outer work and needs load balancing
// for data-dependent sparsity).  With P = softmax(scale q K^T) over the selected
// tokens, o = P V and D = <dO, o> per (query, head):
//   dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Work decomposition on gfx950.  The forward's inverse index is rebuilt (in its
// ordered form): for every (group, block) list, items of at most kBwdItemPairs (query, slot)
// pairs.  A workgroup of four waves (one per SIMD, with up to 512 registers each)
// takes items from per-XCD queues, stages the block's K and V rows in LDS once per
// item and walks the item in sub-chunks of 64 MFMA rows ((64 / G) queries x G
// heads).  Wave w owns keys 32w .. 32w+31 of the block:
//   its K and V slices (B operands of S = Q K^T and dP = dO V^T) and the K^T columns
//   of its dQ dims (A operand of dQ^T = K^T dS^T) are read once per item into AGPRs;
//   per sub-chunk, S and dP for all 64 rows come out with the wave's key on the lane,
//   so P and dS = P (dP - D) are formed in registers and used directly (packed to
//   bf16) as the A operands of dV += P^T dO and dK += dS^T Q, which accumulate in
//   AGPRs over the whole item (32 keys x 128 dims each);
//   dS goes to LDS, and each wave then computes dQ for all 64 rows and dims
//   32w .. 32w+31 over the 128 keys.
// The q and dO rows of a sub-chunk sit in LDS row-major (double-buffered, the next
// sub-chunk's rows loaded during the current one); operands that need them
// transposed use gfx950's transposing LDS read.  LDS layouts are chosen so that
// every access pattern of the loop is free of bank conflicts.  The two 32-row tiles
// are staggered so that the VALU work of one (P, dS) issues between the MFMAs of the
// other.
// dQ leaves as one bf16 partial row per (query, slot, head), summed over the slots
// in fp32 by a second kernel; dK and dV leave as one fp32 partial block per item, summed in
// item order per (group, block) by a third.  No atomics touch a gradient, and the
// inverse index is built in its ordered form (each list's pairs in (query, slot)
// order), so dq, dK and dV are bitwise reproducible for a given workspace size.
#include <type_traits>

#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {

namespace {

constexpr int kBwdRows = 64;  // MFMA rows per sub-chunk
constexpr int kBwdMaxPairs = kBwdItemPairs;  // pairs per item

__device__ __forceinline__ u32x4_t pack8(const float* x) {
  return u32x4_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                 pack_bf16x2(x[6], x[7])};
}

// D[row] = <dO[row], o[row]> over the 128 dims, 16 lanes per row.
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const uint16_t* __restrict__ dO, const float* __restrict__ o,
                                                         int64_t rows, float* __restrict__ D) {
  const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int l = threadIdx.x & 15;
  float acc = 0.f;
  if (row < rows) {
    const u32x4_t g = *reinterpret_cast<const u32x4_t*>(dO + row * kDh + l * 8);
    const float4 a = *reinterpret_cast<const float4*>(o + row * kDh + l * 8);
    const float4 c = *reinterpret_cast<const float4*>(o + row * kDh + l * 8 + 4);
    auto lo = [](uint32_t w) { return __uint_as_float(w << 16); };
    auto hi = [](uint32_t w) { return __uint_as_float(w & 0xffff0000u); };
    acc = lo(g.x) * a.x + hi(g.x) * a.y + lo(g.y) * a.z + hi(g.y) * a.w + lo(g.z) * c.x + hi(g.z) * c.y +
          lo(g.w) * c.z + hi(g.w) * c.w;
  }
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) acc += __shfl_xor(acc, m);
  if (row < rows && l == 0) D[row] = acc;
}

constexpr int kBwdThreads = 256;

// A block's rows (K or V) -> LDS in natural order: row rho (256 B) holds key rho,
// 16-byte chunk c at position c ^ (rho & 15); rows past `nvalid` read as zero.
// 256 threads.
__device__ __forceinline__ void bwd_stage_rows(const uint16_t* __restrict__ src, int row_stride, int nvalid,
                                               uint8_t* T, int tid) {
  const int c = tid & 15;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int rho = (tid >> 4) + 16 * m;
    const int kr = rho < nvalid ? rho : nvalid - 1;
    u32x4_t val = *reinterpret_cast<const u32x4_t*>(src + kr * row_stride + c * 8);
    if (rho >= nvalid) val = u32x4_t{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4_t*>(T + rho * 256 + ((c ^ (rho & 15)) << 4)) = val;
  }
}

// gfx950's transposing LDS read (ds_read_b64_tr_b16) of the 8 bytes at p: within each
// group of 16 lanes, lane i receives element i % 4 of the 8 bytes read by lane
// 4k + i / 4 as its element k (k = 0..3).
__device__ __forceinline__ u32x2_t lds_tr8(const uint8_t* p) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (v4i16 __attribute__((address_space(3)))*)(const_cast<uint8_t*>(p)));
  return __builtin_bit_cast(u32x2_t, x);
}

// Rows R0 .. R0+3 of one column of a row-major tile (rows of 256 B, chunk c of row R
// at (c ^ (R & 15)) * 16): lane i of each 16-lane group (gi = i) receives column
// d0 + i, or d0 + swap23(i) with SW.  Lane j reads 4 columns of row R0 + j / 4.
template <bool SW>
__device__ __forceinline__ u32x2_t tile_tr(const uint8_t* T, int R0, int d0, int gi) {
  const int R = R0 + (gi >> 2);
  const int qd = gi & 3;
  const int col = d0 + 4 * (SW ? ((qd >> 1) | ((qd & 1) << 1)) : qd);
  return lds_tr8(T + R * 256 + (((col >> 3) ^ (R & 15)) << 4) + (col & 7) * 2);
}

// Row tiles of the 4-wave kernel (q and dO rows of a sub-chunk): 16-byte chunk c of
// row R at position c ^ rot2(R % 16), rot2 swapping the two bit pairs.  Sixteen
// consecutive rows at one chunk land in sixteen positions (row-operand reads), and so
// do four consecutive rows at four consecutive chunks (the transposing reads, whose
// 32 lanes then hit 32 distinct 8-byte bank slots).
__device__ __forceinline__ int bwd_row_chunk(int c, int R) { return c ^ (((R & 3) << 2) | ((R >> 2) & 3)); }

// dS of a 64-row sub-chunk, key-major: key K owns 128 bytes, rows in 8-byte runs of
// four (R / 4), run u of key K at slot u ^ g((K / 2) % 16), g rotating the four bits
// right by one.  The 8-byte stores of 32 consecutive keys (one run each) and the
// transposing reads of dQ (4 keys x 8 runs) each hit 32 distinct bank slots.
__device__ __forceinline__ int bwd_ds_offset(int K, int R) {
  const int x = (K >> 1) & 15;
  const int gx = ((x & 1) << 3) | (x >> 1);
  return K * 128 + (((R >> 2) ^ gx) << 3) + (R & 3) * 2;
}

// One wave per SIMD: wave w owns keys 32w .. 32w+31 of the block for S, dP, dV and dK
// (all 64 rows of a sub-chunk, all 128 dims), and dims 32w .. 32w+31 of dQ.  The
// block's K and V slices (B operands of S and dP) and the K^T columns of its dQ dims
// (A operand of dQ^T) are read from LDS once per item into registers, so a sub-chunk
// reads from LDS only its q and dO rows (for S, dP, dV, dK) and dS (for dQ); P and dS
// never leave the wave that formed them except dS for dQ.  The next sub-chunk's q and
// dO rows are loaded straight into the other LDS buffer (16-byte global-to-LDS loads)
// while the current one is computed.
template <int G>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Drow,
    const int4* __restrict__ items, const int32_t* __restrict__ n_items_ptr, const int32_t* __restrict__ pairs,
    int64_t N, int H_kv, int bk, int kk, int64_t w0, float scale, float scale_log2, uint16_t* __restrict__ dq_part,
    uint16_t* __restrict__ dq_dummy, float* __restrict__ dkv_part, int32_t* __restrict__ ctr,
    uint64_t* __restrict__ clk) {
  static_assert(G <= 32, "a sub-chunk holds at least two queries");
  constexpr int kQS = kBwdRows / G;  // queries per sub-chunk
  // 2 x 32 KB block rows + 2 x 2 x 16 KB q/dO rows + 16 KB dS + 3 KB of row tables and
  // the item's pairs: 147 KB (one workgroup per CU).
  __shared__ __attribute__((aligned(16))) uint8_t Ks[kBk * 256];
  __shared__ __attribute__((aligned(16))) uint8_t Vs[kBk * 256];
  __shared__ __attribute__((aligned(16))) uint8_t Qs[2][kBwdRows * 256];
  __shared__ __attribute__((aligned(16))) uint8_t dOs[2][kBwdRows * 256];
  __shared__ __attribute__((aligned(16))) uint8_t dSs[kBk * 128];  // key-major (bwd_ds_offset)
  // Per-row values of a sub-chunk (double-buffered like the rows): lse in base 2, D,
  // the last visible key offset (-1: none) and the row's pair (-1: past the end).
  __shared__ __attribute__((aligned(16))) float rl2[2][kBwdRows];
  __shared__ __attribute__((aligned(16))) float rD[2][kBwdRows];
  __shared__ __attribute__((aligned(16))) int rlim[2][kBwdRows];
  __shared__ __attribute__((aligned(16))) int rprv[2][kBwdRows];
  __shared__ int ipair[kBwdMaxPairs];  // the item's pairs
  __shared__ int64_t wg_item;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int H_q = H_kv * G;
  // Lane-derived addresses are recomputed in each phase from a copy of the lane id the
  // compiler cannot see through, rather than hoisted and held across the loops (which
  // spilled: every unrolled access's address stayed live).
  auto lane_v = [&]() {
    int x = tid & 63;
    asm volatile("" : "+v"(x));
    return x;
  };
  const int lane = tid & 63;
  // Lane parts of the sub-chunk phases' LDS addresses, fixed for the kernel (the
  // k-step, row tile and buffer parts are immediate offsets):
  //   off_s[t]: S/dP operand row l32, chunk 2t + h of a row tile;
  //   off_dvk[dt][run]: dV/dK transposing read of rows 4h + gi/4 + 8 run, dims
  //     32 dt + (l32 & 16) + 4 (gi % 4) .. + 3 (the R % 16 of every row tile's run);
  //   off_dq[tp][nt][s]: dQ transposing read of dS keys 16 tp + 8h + 4s + gi/4
  //     (k-steps of parity tp; two k-steps apart keys differ by 32, 4 KB), rows
  //     32 nt + (l32 & 16) + 4 (gi % 4) .. + 3.
  int off_s[8], off_dvk[4][2], off_dq[2][2][2];
  {
    const int h = lane >> 5, l32 = lane & 31, gi = lane & 15;
#pragma unroll
    for (int t = 0; t < 8; ++t) off_s[t] = l32 * 256 + (bwd_row_chunk(2 * t + h, l32) << 4);
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int run = 0; run < 2; ++run) {
        const int R = 4 * h + (gi >> 2) + 8 * run;
        const int col = 32 * dt + (l32 & 16) + 4 * (gi & 3);
        off_dvk[dt][run] = R * 256 + (bwd_row_chunk(col >> 3, R) << 4) + (col & 7) * 2;
      }
    }
#pragma unroll
    for (int tp = 0; tp < 2; ++tp) {
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
        for (int sr = 0; sr < 2; ++sr)
          off_dq[tp][nt][sr] =
              bwd_ds_offset(16 * tp + 8 * h + 4 * sr + (gi >> 2), 32 * nt + (l32 & 16) + 4 * (gi & 3));
      }
    }
  }
  const int n_items = *n_items_ptr;
  ItemQueue queue{ctr, n_items, (int)gridDim.x, (int)gridDim.x >> 3, (int)(blockIdx.x & 7), kItemCounterStride, 0};
  wg_clock_start(clk);
  if (tid == 0) publish_item(&wg_item, queue.resolve(queue.take()));
  for (;;) {
    __syncthreads();  // the item is published; the previous item's LDS reads are done
    const int64_t item = wg_item;
    if (item < 0) break;
    int ticket = 0;
    if (tid == 0) ticket = queue.take();  // the next item's ticket, in flight meanwhile
    const int4 it = items[item];
    const int64_t b = it.x;
    const int r = it.w;
    const int start = it.y, cnt = it.z;
    // The item's pairs go to LDS with its block (index idx of the item: ipair[idx], idx
    // clamped to cnt - 1).
    static_assert(kBwdMaxPairs % kBwdThreads == 0, "whole rounds of one pair per thread");
    for (int j = tid; j < cnt; j += kBwdThreads) ipair[j] = pairs[start + j];
    auto pair_at = [&](int idx) { return ipair[idx < cnt ? idx : cnt - 1]; };
    __syncthreads();  // the item's pairs
    // q and dO rows of the sub-chunk starting at pair cbase: row rho is (pair
    // cbase + rho / G, head rho % G); thread t fetches 16-byte chunk t % 16 of rows
    // t / 16 + 16 j (j = 0..3) into registers (qv, gv), which go to an LDS buffer at
    // the start of the sub-chunk that uses them.  (Loads straight to LDS would save the
    // registers, but while one is in flight the compiler waits for every LDS read in
    // full, which serialised the MFMA operand fetches.)
    u32x4_t qv[4], gv[4];
    // The next sub-chunk's per-row values (lane L: row L).
    float nx_lse = 0.f, nx_D = 0.f;
    int nx_prv = -1, nx_lim = -1;
    auto fetch_rows = [&](int cbase) {
      const int lv = lane_v();
      const int c = lv & 15;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rho = 4 * wave + (lv >> 4) + 16 * j;
        const int pr = pair_at(cbase + rho / G);
        const int64_t src = ((w0 + (pr >> 5)) * H_q + r * G + rho % G) * kDh + c * 8;
        qv[j] = *reinterpret_cast<const u32x4_t*>(q + src);
        gv[j] = *reinterpret_cast<const u32x4_t*>(dO + src);
      }
    };
    auto store_rows = [&](int buf) {
      const int lv = lane_v();
      const int c = lv & 15;
      if (wave == 0) {
        rl2[buf][lv] = nx_lse * kLog2e;
        rD[buf][lv] = nx_D;
        rlim[buf][lv] = nx_lim;
        rprv[buf][lv] = nx_prv;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rho = 4 * wave + (lv >> 4) + 16 * j;
        *reinterpret_cast<u32x4_t*>(&Qs[buf][rho * 256 + (bwd_row_chunk(c, rho) << 4)]) = qv[j];
        *reinterpret_cast<u32x4_t*>(&dOs[buf][rho * 256 + (bwd_row_chunk(c, rho) << 4)]) = gv[j];
      }
    };
    // Per-row values of a sub-chunk (lane L: row L), written to the row tables by wave 0
    // with the rows.
    auto fetch_info = [&](int cbase) {
      const int my_r = lane_v();
      const int my_idx = cbase + my_r / G;
      const bool my_valid = my_idx < cnt;
      const int my_pr = pair_at(my_idx);
      const int64_t my_row = (w0 + (my_pr >> 5)) * H_q + r * G + my_r % G;
      nx_lse = lse[my_row];
      nx_D = Drow[my_row];
      nx_prv = my_valid ? my_pr : -1;
      // A listed pair's query sees at least key 0 of the block: 0 <= lim; keys past
      // the block (bk = 64) are excluded with it.
      const int64_t lim = w0 + (my_pr >> 5) - b * bk;
      nx_lim = my_valid ? (int)(lim < bk - 1 ? lim : bk - 1) : -1;
    };
    fetch_rows(0);
    fetch_info(0);
    {
      const int64_t tok0 = b * bk;
      const int nvalid = (N - tok0 < bk) ? (int)(N - tok0) : bk;
      const int64_t base = tok0 * H_kv * kDh + (int64_t)r * kDh;
      bwd_stage_rows(kp + base, H_kv * kDh, nvalid, Ks, tid);
      bwd_stage_rows(vp + base, H_kv * kDh, nvalid, Vs, tid);
    }
    __syncthreads();  // K and V rows staged
    // The item's register operands.  kop[t] / vop[t]: dims 16t + 8h .. +7 of key
    // 32w + l32 (B operands of S = Q K^T and dP = dO V^T).  ktop[t]: keys 16t + 8h ..
    // +7 of dim 32w + swap23(l32) (A operand of dQ^T = K^T dS^T; the swap makes a
    // lane's dQ values two runs of 8 consecutive dims).
    u32x4_t kop[8], vop[8], ktop[8];
    {
      const int lv = lane_v();
      const int h = lv >> 5, l32 = lv & 31, gi = lv & 15;
      const int krow = 32 * wave + l32;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int c = 2 * t + h;
        kop[t] = *reinterpret_cast<const u32x4_t*>(Ks + krow * 256 + ((c ^ (krow & 15)) << 4));
        vop[t] = *reinterpret_cast<const u32x4_t*>(Vs + krow * 256 + ((c ^ (krow & 15)) << 4));
        const u32x2_t lo = tile_tr<true>(Ks, 16 * t + 8 * h, 32 * wave + (l32 & 16), gi);
        const u32x2_t hi = tile_tr<true>(Ks, 16 * t + 8 * h + 4, 32 * wave + (l32 & 16), gi);
        ktop[t] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      }
      // The item's operands are held in AGPRs (MFMAs read A and B from either file),
      // which leaves the VGPRs to the sub-chunk's working set.
#pragma unroll
      for (int t = 0; t < 8; ++t) asm volatile("" : "+a"(kop[t]), "+a"(vop[t]), "+a"(ktop[t]));
    }
    f32x16_t dv_acc[4], dk_acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) dv_acc[dt] = dk_acc[dt] = f32x16_t{};

    int cbuf = 0;
    for (int cb = 0; cb < cnt; cb += kQS, cbuf ^= 1) {
      // The sub-chunk's rows go to LDS buffer cbuf (last read two sub-chunks ago);
      // after the barrier all are there, and the previous sub-chunk's dS is free.
      store_rows(cbuf);
      __syncthreads();
      const uint8_t* Qb = Qs[cbuf];
      const uint8_t* dOb = dOs[cbuf];

      // S and dP per 32-row tile rt: element v of tile rt is row rt*32 + 8(v/4) + 4h +
      // v%4, key 32w + l32.  P and dS are formed in registers; packed to bf16 they are
      // the A operands of dV and dK (Pp[rt][s2]: elements 8 s2 .. 8 s2 + 7 of tile rt),
      // and dS goes to LDS for dQ.  The phases are staggered by row tile so that the
      // VALU work of one tile (P, dS) issues between the MFMAs of the other:
      //   S/dP(0); S/dP(1) with P/dS(0); dV/dK(0) with P/dS(1); dV/dK(1).
      // Each step ends in a scheduling barrier, which fixes that interleaving and keeps
      // every operand load one step ahead of its MFMA.
      const int lv = lane_v();
      const int hh = lv >> 5;
      const int key = 32 * wave + (lv & 31);  // this lane's key (offset in the block)
      f32x16_t sacc[2], pacc[2];
      u32x4_t Pp[2][2], dSp[2][2];
      u32x4_t aq[2], ag[2];
      auto sdp_load = [&](int rt, int t) {
        aq[t & 1] = *reinterpret_cast<const u32x4_t*>(Qb + rt * 8192 + off_s[t]);
        ag[t & 1] = *reinterpret_cast<const u32x4_t*>(dOb + rt * 8192 + off_s[t]);
      };
      auto sdp_mfma = [&](int rt, int t) {
        sacc[rt] = mfma_32x32x16(as_bf16x8(aq[t & 1]), as_bf16x8(kop[t]), sacc[rt]);
        pacc[rt] = mfma_32x32x16(as_bf16x8(ag[t & 1]), as_bf16x8(vop[t]), pacc[rt]);
      };
      // Row values of rows rt*32 + 8g + 4h .. +3 (elements 4g .. 4g+3), one broadcast
      // read each, and the elements' P and dS.
      float4 tl2[2], tD[2];
      int4 tlim[2];
      float P[16], dS[16];
      auto pds_load = [&](int rt, int g) {
        const int R = rt * 32 + 8 * g + 4 * hh;
        tl2[g & 1] = *reinterpret_cast<const float4*>(&rl2[cbuf][R]);
        tD[g & 1] = *reinterpret_cast<const float4*>(&rD[cbuf][R]);
        tlim[g & 1] = *reinterpret_cast<const int4*>(&rlim[cbuf][R]);
      };
      auto pds_elem = [&](int rt, int v) {
        const int g = v >> 2, j = v & 3;
        const float4& l4 = tl2[g & 1];
        const float4& d4 = tD[g & 1];
        const int4& m4 = tlim[g & 1];
        const float l2 = j == 0 ? l4.x : j == 1 ? l4.y : j == 2 ? l4.z : l4.w;
        const float Dv = j == 0 ? d4.x : j == 1 ? d4.y : j == 2 ? d4.z : d4.w;
        const int lim = j == 0 ? m4.x : j == 1 ? m4.y : j == 2 ? m4.z : m4.w;
        // Masked rows and keys (past the item's end, or after the query) get 2^-inf
        // = 0; the mask is added to the argument so that nothing here is conditional.
        const float mask = key <= lim ? 0.f : -__builtin_inff();
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[rt][v], scale_log2, -l2) + mask);
        P[v] = p;
        dS[v] = p * (pacc[rt][v] - Dv);
      };
      auto pds_pack = [&](int rt) {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          Pp[rt][s2] = pack8(&P[8 * s2]);
          dSp[rt][s2] = pack8(&dS[8 * s2]);
        }
      };
      // dV += P^T dO and dK += dS^T Q for row tile rt: MFMA rows are the wave's keys;
      // k-slot (h, j) of step (rt, s2) is row rt*32 + 16 s2 + 8(j/4) + 4h + j%4, whose
      // dO and q values come from the row tiles by transposing reads (two runs of four
      // rows).  MFMA i of a tile: s2 = i / 8, dim tile dt = (i / 2) % 4, dK if i is odd.
      constexpr int kDvkAhead = 4;
      u32x4_t bop[kDvkAhead + 1];
      auto dvk_load = [&](int rt, int i) {
        const int s2 = i >> 3, dt = (i >> 1) & 3;
        const uint8_t* tile = (i & 1) ? Qb : dOb;
        const int imm = (rt * 32 + 16 * s2) * 256;
        const u32x2_t lo = lds_tr8(tile + imm + off_dvk[dt][0]);
        const u32x2_t hi = lds_tr8(tile + imm + off_dvk[dt][1]);
        bop[i % (kDvkAhead + 1)] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
      };
      auto dvk_mfma = [&](int rt, int i) {
        const int s2 = i >> 3, dt = (i >> 1) & 3;
        const u32x4_t& bb = bop[i % (kDvkAhead + 1)];
        if (i & 1)
          dk_acc[dt] = mfma_32x32x16(as_bf16x8(dSp[rt][s2]), as_bf16x8(bb), dk_acc[dt]);
        else
          dv_acc[dt] = mfma_32x32x16(as_bf16x8(Pp[rt][s2]), as_bf16x8(bb), dv_acc[dt]);
      };

      // S/dP(0).
      sacc[0] = pacc[0] = sacc[1] = pacc[1] = f32x16_t{};
      sdp_load(0, 0);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (t + 1 < 8) sdp_load(0, t + 1);
        sdp_mfma(0, t);
        __builtin_amdgcn_sched_barrier(0);
      }
      // S/dP(1) with P/dS(0): two elements per k-step.
      sdp_load(1, 0);
      pds_load(0, 0);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        if (t + 1 < 8) sdp_load(1, t + 1);
        if ((t & 1) == 0 && t + 2 < 8) pds_load(0, t / 2 + 1);
        sdp_mfma(1, t);
        pds_elem(0, 2 * t);
        pds_elem(0, 2 * t + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
      pds_pack(0);
      // dV/dK(0) with P/dS(1): one element per MFMA.
      pds_load(1, 0);
#pragma unroll
      for (int i = 0; i < kDvkAhead; ++i) dvk_load(0, i);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i + kDvkAhead < 16) dvk_load(0, i + kDvkAhead);
        if ((i & 3) == 0 && i + 4 < 16) pds_load(1, i / 4 + 1);
        dvk_mfma(0, i);
        pds_elem(1, i);
        __builtin_amdgcn_sched_barrier(0);
      }
      pds_pack(1);
      // dS into dSs key-major: the lane's key holds four runs of four consecutive rows
      // per tile, one 8-byte store each.
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const u32x4_t& src = dSp[rt][g >> 1];
          *reinterpret_cast<u32x2_t*>(dSs + bwd_ds_offset(key, rt * 32 + 8 * g + 4 * hh)) =
              (g & 1) ? u32x2_t{src[2], src[3]} : u32x2_t{src[0], src[1]};
        }
      }
      // The next sub-chunk's rows are fetched from here on (not earlier, so that their
      // registers are free during S/dP and P/dS).
      if (cb + kQS < cnt) {
        fetch_rows(cb + kQS);
        fetch_info(cb + kQS);
      }
      __syncthreads();  // dS complete
      // dV/dK(1) and dQ^T = K^T dS^T as one sequence, their MFMAs alternating (each with
      // its operand reads a few steps ahead), so that neither waits alone on its LDS
      // reads.  dQ: rows 32 nt + l32 (MFMA columns), dims 32w + swap23(i) (MFMA rows),
      // all 128 keys; its dS^T operand by transposing reads of the key-major dS: lane L
      // of a group reads rows rb .. rb+3 of key K0 + L / 4, so lane i receives row
      // (group's first row) + i of keys K0 .. K0+3.
      {
        constexpr int kDqAhead = 4;
        u32x4_t sop[16];
        // dQ MFMA i: k-step t = i / 2 of row tile nt = i % 2.
        auto load_s = [&](int i) {
          const int t = i >> 1, nt = i & 1;
          const u32x2_t lo = lds_tr8(dSs + 4096 * (t >> 1) + off_dq[t & 1][nt][0]);
          const u32x2_t hi = lds_tr8(dSs + 4096 * (t >> 1) + off_dq[t & 1][nt][1]);
          sop[i] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        };
        f32x16_t qacc[2];
        qacc[0] = qacc[1] = f32x16_t{};
#pragma unroll
        for (int i = 0; i < kDvkAhead; ++i) dvk_load(1, i);
#pragma unroll
        for (int i = 0; i < kDqAhead; ++i) load_s(i);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (i + kDvkAhead < 16) dvk_load(1, i + kDvkAhead);
          dvk_mfma(1, i);
          __builtin_amdgcn_sched_barrier(0);
          if (i + kDqAhead < 16) load_s(i + kDqAhead);
          qacc[i & 1] = mfma_32x32x16(as_bf16x8(ktop[i >> 1]), as_bf16x8(sop[i]), qacc[i & 1]);
          __builtin_amdgcn_sched_barrier(0);
        }
        // dQ rows (bf16, one per pair and head, scaled): element v of lane (l32, h) in
        // tile nt is row 32 nt + l32, dim 32w + 8h + 16(v / 8) + v % 8.  Rows past the
        // item's end write to a dummy row, so every lane stores and the count of
        // stores (which the next sub-chunk's wait for its row loads must not cover) is
        // fixed.
        const int lv = lane_v();
        const int h = lv >> 5, l32 = lv & 31;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int row = 32 * nt + l32;
          const int pr = rprv[cbuf][row];
          const int64_t prow = (((int64_t)(pr >> 5) * H_kv + r) * kk + (pr & 31)) * G + row % G;
          uint16_t* dst = pr >= 0 ? dq_part + prow * kDh + 32 * wave + 8 * h : dq_dummy;
#pragma unroll
          for (int run = 0; run < 2; ++run) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = qacc[nt][8 * run + e] * scale;
            *reinterpret_cast<u32x4_t*>(dst + 16 * run) = pack8(x);
          }
        }
      }
    }
    // The item's dK (scaled) and dV: element v of lane (l32, h) in dim tile dt is key
    // 32w + 8(v/4) + 4h + v%4, dim 32dt + l32.
    {
    const int lv = lane_v();
    const int h = lv >> 5, l32 = lv & 31;
    float* kpart = dkv_part + item * 2 * (kBk * kDh);
    float* vpart = kpart + kBk * kDh;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int kx = 32 * wave + 8 * (v >> 2) + 4 * h + (v & 3);
        kpart[kx * kDh + 32 * dt + l32] = dk_acc[dt][v] * scale;
        vpart[kx * kDh + 32 * dt + l32] = dv_acc[dt][v];
      }
    }
    }
    if (tid == 0) publish_item(&wg_item, queue.resolve(ticket));  // read by all after the next barrier
  }
  wg_clock_end(clk);
}

// dQ: per (query, head) the sum of its valid slots' partial rows in slot order; 16
// lanes per row, 8 dims (16 bytes of each partial row) each.  The valid slots are listed first so that the row
// loads can be issued four at a time.
__global__ __launch_bounds__(256) void bwd_dq_combine_kernel(const uint16_t* __restrict__ dq_part,
                                                             const int32_t* __restrict__ block_idx, int64_t w0,
                                                             int64_t W, int H_kv, int G, int kk, int bsh,
                                                             float* __restrict__ dq) {
  const int64_t gr = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;  // (query in window, head)
  const int l = threadIdx.x & 15;
  const int H_q = H_kv * G;
  if (gr >= W * H_q) return;
  const int64_t il = gr / H_q;
  const int hh = (int)(gr % H_q);
  const int r = hh / G, g = hh % G;
  const int64_t i = w0 + il;
  const int32_t* sel = block_idx + (i * H_kv + r) * kk;
  uint32_t vmask = 0;  // kk <= 32
  for (int s = 0; s < kk; ++s) {
    const int bb = sel[s];
    if (bb >= 0 && (int64_t)bb <= (i >> bsh)) vmask |= 1u << s;
  }
  const uint16_t* base = dq_part + ((il * H_kv + r) * kk * G + g) * kDh + 8 * l;
  const int64_t sstride = (int64_t)G * kDh;  // elements between consecutive slots' rows
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](const u32x4_t& x) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      acc[2 * m] += __uint_as_float(x[m] << 16);
      acc[2 * m + 1] += __uint_as_float(x[m] & 0xffff0000u);
    }
  };
  while (vmask) {
    int sl[4];
    int n = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sl[j] = vmask ? __builtin_ctz(vmask) : -1;
      if (vmask) {
        vmask &= vmask - 1;
        ++n;
      }
    }
    u32x4_t x[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      x[j] = *reinterpret_cast<const u32x4_t*>(base + (sl[j] < 0 ? sl[0] : sl[j]) * sstride);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < n) add(x[j]);
  }
  float* out = dq + (i * H_q + hh) * kDh + 8 * l;
  *reinterpret_cast<float4*>(out) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *reinterpret_cast<float4*>(out + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// dK, dV of block b, group r: the partial blocks of the items of its lists (one per
// query window), summed in item order and added to dk / dv; a thread sums 4
// consecutive elements, with four items' loads in flight.
__global__ __launch_bounds__(256) void bwd_kv_reduce_kernel(const float* __restrict__ dkv_part,
                                                            const int32_t* __restrict__ counts,
                                                            const int32_t* __restrict__ lfirst, int item_q,
                                                            int64_t B, int bk, int nW, int H_kv, int64_t N,
                                                            float* __restrict__ dk, float* __restrict__ dv) {
  const int64_t rb = blockIdx.x;
  const int r = (int)(rb / B);
  const int64_t b = rb % B;
  constexpr int kBlockElems = kBk * kDh;
  for (int e4 = threadIdx.x; e4 < 2 * kBlockElems / 4; e4 += 256) {
    const int e = 4 * e4;
    const int which = e / kBlockElems, kd = e % kBlockElems;
    const int key = kd / kDh, d = kd % kDh;
    const int64_t tok = b * bk + key;
    if (key >= bk || tok >= N) continue;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    auto add = [&](const float4& x) {
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    };
    for (int w = 0; w < nW; ++w) {
      const int64_t l = ((int64_t)r * nW + w) * B + b;
      const int n = counts[l];
      const int nit = (n + item_q - 1) / item_q;
      const float* src = dkv_part + ((int64_t)lfirst[l] * 2 + which) * kBlockElems + kd;
      constexpr int64_t kItemStride = 2 * kBlockElems;
      int t = 0;
      for (; t + 4 <= nit; t += 4) {
        float4 x[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = *reinterpret_cast<const float4*>(src + (t + j) * kItemStride);
#pragma unroll
        for (int j = 0; j < 4; ++j) add(x[j]);
      }
      for (; t < nit; ++t) add(*reinterpret_cast<const float4*>(src + t * kItemStride));
    }
    float* out = (which ? dv : dk) + (tok * H_kv + r) * kDh + d;
    float4 o4 = *reinterpret_cast<float4*>(out);
    o4.x += acc.x;
    o4.y += acc.y;
    o4.z += acc.z;
    o4.w += acc.w;
    *reinterpret_cast<float4*>(out) = o4;
  }
}

__global__ void bwd_zero_kernel(float* __restrict__ p, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) p[e] = 0.f;
}

}  // namespace

hipError_t launch_bwd_prepare(const uint16_t* dO, const float* o, int64_t rows, float* D, float* dk, float* dv,
                              int64_t kv_elems, hipStream_t stream) {
  bwd_rowdot_kernel<<<dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, stream>>>(dO, o, rows, D);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  bwd_zero_kernel<<<dim3(1024), dim3(256), 0, stream>>>(dk, kv_elems);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwd_zero_kernel<<<dim3(1024), dim3(256), 0, stream>>>(dv, kv_elems);
  return hipGetLastError();
}

hipError_t launch_bwd_window(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dO,
                             const float* lse, const float* D, const int32_t* block_idx, int64_t N, int64_t B,
                             int bk, int H_q, int H_kv, int kk, float scale, int64_t w0, int64_t W, int num_cus,
                             float* dq, float* dk, float* dv, uint8_t* ws, const AttnWorkspace& L,
                             hipStream_t stream, uint64_t* clk) {
  const int G = H_q / H_kv;
  const int bsh = bk == 64 ? 6 : 7;
  int32_t* lfirst = reinterpret_cast<int32_t*>(ws + L.lfirst);
  hipError_t e = launch_inverse_index(block_idx, B, SeqInfo{}, bsh, H_kv, kk, w0, W, ws, L, stream, lfirst,
                                      /*ordered=*/true);
  if (e != hipSuccess) return e;
  const int32_t* n_items = reinterpret_cast<const int32_t*>(ws + L.n_items);
  const int4* items = reinterpret_cast<const int4*>(ws + L.items);
  const int32_t* pairs = reinterpret_cast<const int32_t*>(ws + L.pairs);
  const int32_t* counts = reinterpret_cast<const int32_t*>(ws + L.counts);
  uint16_t* dq_part = reinterpret_cast<uint16_t*>(ws + L.opart);
  // One row past the (pair, head) rows: where rows past an item's end write.
  uint16_t* dq_dummy = dq_part + (int64_t)W * H_kv * kk * G * kDh;
  float* dkv_part = reinterpret_cast<float*>(ws + L.lpart);
  int32_t* ctr = reinterpret_cast<int32_t*>(ws + L.ctr);
  int64_t grid = num_cus;
  if (grid > L.max_items) grid = L.max_items;
  grid = ((grid + 7) / 8) * 8;
  const float scale_log2 = scale * kLog2e;
  switch (G) {
#define MSA_BWD_CASE(GG)                                                                                  \
  case GG:                                                                                                \
    bwd_kernel<GG><<<dim3((unsigned)grid), dim3(kBwdThreads), 0, stream>>>(                              \
        q, k, v, dO, lse, D, items, n_items, pairs, N, H_kv, bk, kk, w0, scale, scale_log2, dq_part, dq_dummy, \
        dkv_part, ctr, clk);                                                                              \
    break;
    MSA_BWD_CASE(1)
    MSA_BWD_CASE(2)
    MSA_BWD_CASE(4)
    MSA_BWD_CASE(8)
    MSA_BWD_CASE(16)
    MSA_BWD_CASE(32)
#undef MSA_BWD_CASE
    default:
      return hipErrorInvalidValue;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t rows = W * H_q;
  bwd_dq_combine_kernel<<<dim3((unsigned)((rows * 16 + 255) / 256)), dim3(256), 0, stream>>>(
      dq_part, block_idx, w0, W, H_kv, G, kk, bsh, dq);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  bwd_kv_reduce_kernel<<<dim3((unsigned)(H_kv * B)), dim3(256), 0, stream>>>(dkv_part, counts, lfirst, L.item_q, B,
                                                                             bk, L.nW, H_kv, N, dk, dv);
  return hipGetLastError();
}

}  // namespace msa
