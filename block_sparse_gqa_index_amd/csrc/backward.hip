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
// ordered form): for every (group, block) list, items of at most 256 (query, slot)
// pairs.  A workgroup of eight waves (two per SIMD, so one wave's LDS and memory
// waits overlap the other's work) stages the block's K, V (rows) and K^T in LDS
// once per item and walks the item in sub-chunks of 64 MFMA rows ((64 / G) queries
// x G heads), with the q and dO rows of the sub-chunk in LDS row-major (operands
// that need them transposed use transposing LDS reads).  Wave w owns keys
// 32(w % 4) .. +31 of the block and dims 64(w / 4) .. +63 of its dK and dV:
//   S = Q K^T and dP = dO V^T on 32x32x16 MFMAs give, per lane, one key (the lane)
//   and 32 rows (registers), so P and dS are formed in registers; the two waves of
//   a key slice take one 32-row tile each and hand the other their P through LDS
//   (their dS through the dS rows written for dQ);
//   dV += P^T dO and dK += dS^T Q use P and dS directly as MFMA operands, and
//   accumulate in registers over the whole item (each wave holding half the dims,
//   which is what lets two waves share a SIMD);
//   dS goes to LDS, and each wave then computes dQ for 32 rows x 32 dims over all
//   128 keys (dS K, with K^T as the operand).
// dQ leaves as one bf16 partial row per (query, slot, head), summed over the slots
// in fp32 by a second kernel; dK and dV leave as one fp32 partial block per item, summed in
// item order per (group, block) by a third.  No atomics touch a gradient, and the
// inverse index is built in its ordered form (each list's pairs in (query, slot)
// order), so dq, dK and dV are bitwise reproducible for a given workspace size.
#include <utility>

#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {

namespace {

constexpr int kBwdThreads = 512;
constexpr int kBwdRows = 64;  // MFMA rows per sub-chunk
constexpr int kBwdPairRegs = 4;  // an item holds at most 256 pairs: 4 registers of 64 lanes

// Pair idx of the item (any lane): register idx / 64 of lane idx % 64.
__device__ __forceinline__ int bwd_pair_at(const int (&ip)[kBwdPairRegs], int idx) {
  int v = 0;
#pragma unroll
  for (int k = 0; k < kBwdPairRegs; ++k) {
    const int x = __shfl(ip[k], idx & 63);
    v = (idx >> 6) == k ? x : v;
  }
  return v;
}

__device__ __forceinline__ u32x4_t pack8(const float* x) {
  return u32x4_t{pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                 pack_bf16x2(x[6], x[7])};
}

// dS of a sub-chunk in LDS, key-major: key K (0..127) owns 128 bytes, rows 0..63 as
// bf16, in 16-byte chunks of 8 rows placed at chunk (R / 8) ^ (K % 8), so that the
// 8-byte accesses of one instruction (consecutive keys) spread over the banks.  Runs
// of four rows starting at a multiple of 4 stay inside one chunk.
__device__ __forceinline__ int bwd_ds_offset(int K, int R) { return K * 128 + ((((R >> 3) ^ K) & 7) << 4) + (R & 7) * 2; }

// Per-row values of a 64-row sub-chunk are kept one row per lane, row R on lane
// bwd_row_lane(R): bit 2 of R picks the lane half and the other five bits the lane
// within it.  The S/dP layout needs, in lane half h, rows whose bit 2 is h, so each
// such read is a broadcast of one lane within the reader's own half.
__device__ __forceinline__ int bwd_row_lane(int R) { return (((R >> 2) & 1) << 5) | (R & 3) | ((R >> 3) << 2); }
__device__ __forceinline__ int bwd_lane_row(int L) { return (L & 3) | (((L >> 5) & 1) << 2) | (((L >> 2) & 7) << 3); }

// Broadcast lane M of each 32-lane half (ds_swizzle, bit-mask mode: and 0, or M).
template <int M>
__device__ __forceinline__ int half_bcast(int x) {
  static_assert(M >= 0 && M < 32, "lane within a half");
  return __builtin_amdgcn_ds_swizzle(x, M << 5);
}
template <int M>
__device__ __forceinline__ float half_bcast(float x) {
  return __int_as_float(half_bcast<M>(__float_as_int(x)));
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>), in order.
template <class F, int... V>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, V...>) {
  (f(std::integral_constant<int, V>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
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

template <int G>
__global__ __launch_bounds__(kBwdThreads, 1) void bwd_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
    const uint16_t* __restrict__ dO, const float* __restrict__ lse, const float* __restrict__ Drow,
    const int4* __restrict__ items, const int32_t* __restrict__ n_items_ptr, const int32_t* __restrict__ pairs,
    int64_t N, int H_kv, int64_t B, int bk, int nW, int kk, int64_t w0, float scale, float scale_log2,
    uint16_t* __restrict__ dq_part, float* __restrict__ dkv_part, int32_t* __restrict__ ctr,
    uint64_t* __restrict__ clk) {
  static_assert(G <= 32, "a sub-chunk holds at least two queries");
  constexpr int kQS = kBwdRows / G;  // queries per sub-chunk
  // 3 x 32 KB block tiles + 4 x 16 KB sub-chunk tiles = 160 KB (one workgroup per CU).
  __shared__ __attribute__((aligned(16))) uint8_t Ks[kBk * 256];   // K rows (key swap23(rho) at row rho)
  __shared__ __attribute__((aligned(16))) uint8_t Vs[kBk * 256];   // V rows, same order
  __shared__ __attribute__((aligned(16))) uint8_t Kt[kDh * 256];   // K^T, keys in natural order
  __shared__ __attribute__((aligned(16))) uint8_t Qs[kBwdRows * 256];   // q rows
  __shared__ __attribute__((aligned(16))) uint8_t dOs[kBwdRows * 256];  // dO rows
  __shared__ __attribute__((aligned(16))) uint8_t dSs[kBwdRows * 256];  // dS, key-major (bwd_ds_offset)
  __shared__ __attribute__((aligned(16))) uint8_t Px[8 * 2048];         // each wave's P for its partner

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int ks = wave & 3, dh = wave >> 2;  // key slice, dK/dV dim half
  const int h = lane >> 5, l32 = lane & 31;
  const int H_q = H_kv * G;
  const int n_items = *n_items_ptr;
  // Items from the per-XCD queues (as in the forward kernels); the next item is
  // published through the first 8 bytes of the dS tile, which is free from the
  // item's last barrier until after the next item's first sub-chunk barrier.
  int64_t* const wg_item = reinterpret_cast<int64_t*>(dSs);
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
    const int64_t b = it.x, r = it.w;
    const int start = it.y, cnt = it.z;
    int ip[kBwdPairRegs];
#pragma unroll
    for (int k = 0; k < kBwdPairRegs; ++k) ip[k] = pairs[start + (64 * k + lane < cnt ? 64 * k + lane : cnt - 1)];
    {
      // Threads 0..255 stage K and V rows, threads 256..511 K^T.
      int stid = tid & 255;
      asm volatile("" : "+v"(stid));
      // A block of bk (64 or 128) keys fills the first bk rows of the staged tiles.
      const int64_t tok0 = b * bk;
      const int nvalid = (N - tok0 < bk) ? (int)(N - tok0) : bk;
      const int64_t base = tok0 * H_kv * kDh + r * kDh;
      if (tid < 256) {
        stage_k(kp + base, H_kv * kDh, nvalid, Ks, stid);
        stage_k(vp + base, H_kv * kDh, nvalid, Vs, stid);
      } else {
        stage_v(kp + base, H_kv * kDh, nvalid, Kt, stid);
      }
    }

    f32x16_t dv_acc[2], dk_acc[2];
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) dv_acc[dt] = dk_acc[dt] = f32x16_t{};

    // Row l of a sub-chunk (l = 0..63) is (pair cb + l / G, head l % G); lane l keeps
    // that row's pair (-1: past the item's end), lse, D and last visible key offset
    // within the block (-1: none) for the others to read by shuffles.  Thread t loads
    // 16-byte chunk t & 15 of rows (t >> 4) + 32j of q and dO.  Both are fetched one
    // sub-chunk ahead, so their latency hides under the previous sub-chunk's work.
    u32x4_t qv[2], gv[2];
    int my_prv, my_lim;
    float my_l2, my_D;
    auto fetch = [&](int cbase) {
      const int my_r = bwd_lane_row(lane);  // the row this lane describes
      const int my_idx = cbase + my_r / G;
      const bool my_valid = my_idx < cnt;
      const int my_pr = bwd_pair_at(ip, my_valid ? my_idx : cnt - 1);
      const int64_t my_row = (w0 + (my_pr >> 5)) * H_q + r * G + my_r % G;
      my_l2 = lse[my_row] * kLog2e;
      my_D = Drow[my_row];
      my_prv = my_valid ? my_pr : -1;
      // A listed pair's query sees at least key 0 of the block: 0 <= lim; keys past
      // the block (bk = 64) are excluded with it.
      const int64_t lim = w0 + (my_pr >> 5) - b * bk;
      my_lim = my_valid ? (int)(lim < bk - 1 ? lim : bk - 1) : -1;
      const int c = tid & 15;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int rho = (tid >> 4) + 32 * j;
        const int idx = cbase + rho / G;
        const int pr = bwd_pair_at(ip, idx < cnt ? idx : cnt - 1);
        const int64_t src = ((w0 + (pr >> 5)) * H_q + r * G + rho % G) * kDh + c * 8;
        qv[j] = *reinterpret_cast<const u32x4_t*>(q + src);
        gv[j] = *reinterpret_cast<const u32x4_t*>(dO + src);
      }
    };
    fetch(0);

    for (int cb = 0; cb < cnt; cb += kQS) {
      asm volatile("" ::: "memory");
      {
        const int c = tid & 15;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int rho = (tid >> 4) + 32 * j;
          *reinterpret_cast<u32x4_t*>(Qs + rho * 256 + ((c ^ (rho & 15)) << 4)) = qv[j];
          *reinterpret_cast<u32x4_t*>(dOs + rho * 256 + ((c ^ (rho & 15)) << 4)) = gv[j];
        }
      }
      const int cur_prv = my_prv, cur_lim = my_lim;
      const float cur_l2 = my_l2, cur_D = my_D;
      __syncthreads();  // rows staged (and, on the first sub-chunk, the block)
      fetch(cb + kQS < cnt ? cb + kQS : cb);  // the next sub-chunk (past the end: reread, unused)

      // Lane-derived LDS addresses are recomputed in each phase from a copy of the
      // lane id the compiler cannot see through, rather than held across the loop.
      auto lane_v = [&]() {
        int x = lane;
        asm volatile("" : "+v"(x));
        return x;
      };
      // S and dP of this wave's row tile rt = dh (the other tile is its partner's,
      // wave ^ 4, which owns the same keys): element v is row rt*32 + 8(v/4) + 4h + v%4,
      // key koff.  P and dS leave this phase as bf16 MFMA operands: Pp[s2] holds
      // elements 8 s2 .. 8 s2 + 7.
      u32x4_t Pp[2], dSp[2];
      auto s_dp = [&](auto RTC) {
        constexpr int rt = decltype(RTC)::value;
        const int lv = lane_v();
        const int h = lv >> 5, l32 = lv & 31;
        const int krow = 32 * ks + l32;
        const int koff = 32 * ks + swap23(l32);
        f32x16_t sacc = f32x16_t{}, pacc = f32x16_t{};
        const int row = rt * 32 + l32;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int c = 8 * h + t;
          const u32x4_t aq = *reinterpret_cast<const u32x4_t*>(Qs + row * 256 + ((c ^ (row & 15)) << 4));
          const u32x4_t bk = *reinterpret_cast<const u32x4_t*>(Ks + krow * 256 + ((c ^ (krow & 15)) << 4));
          sacc = mfma_32x32x16(as_bf16x8(aq), as_bf16x8(bk), sacc);
          const u32x4_t ag = *reinterpret_cast<const u32x4_t*>(dOs + row * 256 + ((c ^ (row & 15)) << 4));
          const u32x4_t bv = *reinterpret_cast<const u32x4_t*>(Vs + krow * 256 + ((c ^ (krow & 15)) << 4));
          pacc = mfma_32x32x16(as_bf16x8(ag), as_bf16x8(bv), pacc);
        }
        float P[16], dS[16];
        // Element v: row rt*32 + 8(v/4) + 4h + v%4, held by lane v + 16 rt of this
        // lane's half.
        static_for<16>([&](auto VC) {
          constexpr int v = decltype(VC)::value;
          const float l2 = half_bcast<v + 16 * rt>(cur_l2);
          const float Dv = half_bcast<v + 16 * rt>(cur_D);
          const int lim = half_bcast<v + 16 * rt>(cur_lim);
          const bool in = koff <= lim;  // a real row, and causal
          const float p = in ? __builtin_amdgcn_exp2f(fmaf(sacc[v], scale_log2, -l2)) : 0.f;
          P[v] = p;
          dS[v] = p * (pacc[v] - Dv);
        });
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          Pp[s2] = pack8(&P[8 * s2]);
          dSp[s2] = pack8(&dS[8 * s2]);
        }
      };
      if (dh == 0)
        s_dp(std::integral_constant<int, 0>{});
      else
        s_dp(std::integral_constant<int, 1>{});
      // The wave's P goes to Px for its partner (wave w's 2 KB at w * 2 KB, operand s2
      // of lane l at (64 s2 + l) * 16 B); its dS goes into dSs key-major: the lane's key
      // holds the four runs of four consecutive rows of its 16 values, one 8-byte store
      // each.  Both areas were last read before the previous sub-chunk's final barrier.
      {
        const int lv = lane_v();
        const int h = lv >> 5;
        const int koff = 32 * ks + swap23(lv & 31);
        u32x4_t* xp = reinterpret_cast<u32x4_t*>(Px + wave * 2048) + lv;
        xp[0] = Pp[0];
        xp[64] = Pp[1];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int r0 = dh * 32 + 8 * g + 4 * h;  // values v = 4g .. 4g + 3
          const u32x4_t& src = dSp[g >> 1];
          *reinterpret_cast<u32x2_t*>(dSs + bwd_ds_offset(koff, r0)) =
              (g & 1) ? u32x2_t{src[2], src[3]} : u32x2_t{src[0], src[1]};
        }
      }
      __syncthreads();  // P exchanged, dS complete
      // dV += P^T dO and dK += dS^T Q over both row tiles, this wave's first: MFMA rows
      // are the wave's keys (row i holds key 32(w % 4) + swap23(i)); k-slot (h, j) of
      // step (rt, s2) is row rt*32 + 16 s2 + 8(j/4) + 4h + j%4.  The partner's P comes
      // from Px, its dS from the rows in dSs.  The dO and q operands (8 rows of one dim
      // per lane) are read from the row-major tiles with transposing LDS reads: within
      // each group of 16 lanes, lane i receives element i % 4 of the 8 bytes read by
      // lane 4k + i / 4, for k = 0..3; so lane j of a group reads 4 dims 4(j % 4) ..
      // of row R0 + j / 4, and lane i gets rows R0 .. R0+3 of dim i.
      {
        const int lv = lane_v();
        const int h = lv >> 5, l32 = lv & 31;
        const int koff = 32 * ks + swap23(l32);
        const int rto = dh ^ 1;
        const int gi = lv & 15;  // index within the 16-lane group
        // Transposing read of 4 rows R0 .. R0+3 of tile T for dims d0 .. d0+15.
        auto tr4 = [&](const uint8_t* T, int R0, int d0) -> u32x2_t {
          const int R = R0 + (gi >> 2);
          const int col = d0 + 4 * (gi & 3);
          const uint8_t* p = T + R * 256 + ((((col >> 3) ^ (R & 15))) << 4) + (col & 7) * 2;
          typedef short v4i16 __attribute__((ext_vector_type(4)));
          const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (v4i16 __attribute__((address_space(3)))*)(const_cast<uint8_t*>(p)));
          return __builtin_bit_cast(u32x2_t, x);
        };
        u32x4_t Po[2], dSo[2];
        const u32x4_t* xo = reinterpret_cast<const u32x4_t*>(Px + (wave ^ 4) * 2048) + lv;
        Po[0] = xo[0];
        Po[1] = xo[64];
        // The partner's dS at this lane's key: k-slots j = 0..3 and 4..7 of step s2 are
        // the runs of rows rto*32 + 16 s2 + 4h and + 8 (four consecutive rows each).
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int r0 = rto * 32 + 16 * s2 + 4 * h;
          const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(dSs + bwd_ds_offset(koff, r0));
          const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(dSs + bwd_ds_offset(koff, r0 + 8));
          dSo[s2] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
        }
#pragma unroll
        for (int tile = 0; tile < 2; ++tile) {
          const int rt = tile ? rto : dh;
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const u32x4_t ap = tile ? Po[s2] : Pp[s2];
            const u32x4_t ad = tile ? dSo[s2] : dSp[s2];
            const int R0 = rt * 32 + 16 * s2 + 4 * h;
#pragma unroll
            for (int dt = 0; dt < 2; ++dt) {
              const int d0 = 64 * dh + dt * 32 + (l32 & 16);  // this lane group's 16 dims
              const u32x2_t o0 = tr4(dOs, R0, d0), o1 = tr4(dOs, R0 + 8, d0);
              const u32x4_t bo = u32x4_t{o0[0], o0[1], o1[0], o1[1]};
              dv_acc[dt] = mfma_32x32x16(as_bf16x8(ap), as_bf16x8(bo), dv_acc[dt]);
              const u32x2_t q0 = tr4(Qs, R0, d0), q1 = tr4(Qs, R0 + 8, d0);
              const u32x4_t bq = u32x4_t{q0[0], q0[1], q1[0], q1[1]};
              dk_acc[dt] = mfma_32x32x16(as_bf16x8(ad), as_bf16x8(bq), dk_acc[dt]);
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      {
        // dQ^T = K^T dS^T over all 128 keys: wave w takes dQ rows 32(w & 1) + 0..31
        // (MFMA columns, one per lane) and dims 32(w >> 1) + 0..31 (MFMA rows; lane l
        // reads K^T row swap23(l), so a lane's 16 values are the two runs of 8
        // consecutive dims 8h .. 8h+7 and 16+8h .. 16+8h+7 of its dQ row).
        const int lv = lane_v();
        const int h = lv >> 5, l32 = lv & 31;
        const int row = 32 * (wave & 1) + l32;
        const int d = 32 * (wave >> 1) + swap23(l32);
        // The B operand (8 keys of the lane's dQ row) from the key-major dS by
        // transposing reads: in each group of 16 lanes, lane L reads rows
        // Rb + 4(L % 4) .. + 3 of key K0 + L / 4, so lane i receives row Rb + i of keys
        // K0 .. K0 + 3 (Rb: the group's first row).
        const int gl = lv & 15;
        const int rb = 32 * (wave & 1) + (l32 & 16) + 4 * (gl & 3);
        auto ds_tr = [&](int k0) -> u32x2_t {
          typedef short v4i16 __attribute__((ext_vector_type(4)));
          const uint8_t* p = dSs + bwd_ds_offset(k0 + (gl >> 2), rb);
          const v4i16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (v4i16 __attribute__((address_space(3)))*)(const_cast<uint8_t*>(p)));
          return __builtin_bit_cast(u32x2_t, x);
        };
        f32x16_t qacc = f32x16_t{};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int kc = 2 * t + h;
          const u32x4_t ak = *reinterpret_cast<const u32x4_t*>(Kt + d * 256 + ((kc ^ (d & 15)) << 4));
          const u32x2_t s0 = ds_tr(8 * kc), s1 = ds_tr(8 * kc + 4);
          const u32x4_t bs = u32x4_t{s0[0], s0[1], s1[0], s1[1]};
          qacc = mfma_32x32x16(as_bf16x8(ak), as_bf16x8(bs), qacc);
        }
        const int pr = __shfl(cur_prv, bwd_row_lane(row));
        if (pr >= 0) {
          const int64_t prow = (((int64_t)(pr >> 5) * H_kv + r) * kk + (pr & 31)) * G + row % G;
          uint16_t* dst = dq_part + prow * kDh + 32 * (wave >> 1) + 8 * h;
#pragma unroll
          for (int run = 0; run < 2; ++run) {
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = qacc[8 * run + e] * scale;
            *reinterpret_cast<u32x4_t*>(dst + 16 * run) = pack8(x);
          }
        }
      }
      __syncthreads();  // the sub-chunk's LDS tiles may be replaced
    }
    // The item's dK (scaled) and dV: element v of lane (l32, h) is key
    // 32(w % 4) + swap23(8(v/4) + 4h + v%4), dim 64(w / 4) + 32dt + l32.
    float* kpart = dkv_part + item * 2 * (kBk * kDh);
    float* vpart = kpart + kBk * kDh;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = 32 * ks + swap23(8 * (v >> 2) + 4 * h + (v & 3));
        kpart[key * kDh + 64 * dh + 32 * dt + l32] = dk_acc[dt][v] * scale;
        vpart[key * kDh + 64 * dh + 32 * dt + l32] = dv_acc[dt][v];
      }
    }
    if (tid == 0) publish_item(wg_item, queue.resolve(ticket));  // read by all after the next barrier
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
  float* dkv_part = reinterpret_cast<float*>(ws + L.lpart);
  int32_t* ctr = reinterpret_cast<int32_t*>(ws + L.ctr);
  int64_t grid = num_cus;
  if (grid > L.max_items) grid = L.max_items;
  grid = ((grid + 7) / 8) * 8;
  const float scale_log2 = scale * kLog2e;
  switch (G) {
#define MSA_BWD_CASE(GG)                                                                                  \
  case GG:                                                                                                \
    bwd_kernel<GG><<<dim3((unsigned)grid), dim3(kBwdThreads), 0, stream>>>(                                \
        q, k, v, dO, lse, D, items, n_items, pairs, N, H_kv, B, bk, L.nW, kk, w0, scale, scale_log2, dq_part, \
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
