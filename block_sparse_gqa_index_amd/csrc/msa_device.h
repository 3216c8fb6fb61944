// Device-side helpers shared by the MSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
// Native 16- and 8-byte integer vectors (HIP's uint4/uint2 are structs whose
// copies can block promotion of local arrays to registers).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kDh = 128;    // head dim of the main branch
constexpr int kDidx = 64;   // index head dim
constexpr int kBk = 128;    // keys per block
constexpr int kWave = 64;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t u) { return __builtin_bit_cast(bf16x8_t, u); }

// D(32x32) += A(32x16) * B(16x32), bf16 in, fp32 accumulate.
// Lane l supplies A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32]; it receives
// D[8*(v/4) + 4*(l/32) + v%4][l%32] in element v.
__device__ __forceinline__ f32x16_t mfma_32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16) += A(16x32) * B(32x16).  Lane l supplies A[l%16][8*(l/16) .. +7] and
// B[8*(l/16) .. +7][l%16]; it receives D[4*(l/16) + v][l%16] in element v.
__device__ __forceinline__ f32x4_t mfma_16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two fp32 -> packed bf16x2 with round-to-nearest-even (inputs are finite).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
  bf16x2_t v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// ---------------------------------------------------------------------------------
// Streaming Top-L list kept in registers by one lane: values descending, and among
// equal values the lower block index first.  Blocks must be offered in increasing
// index order, so a newcomer ranks below every kept entry of equal value.
template <int L>
struct TopList {
  float v[L];
  int b[L];

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int j = 0; j < L; ++j) {
      v[j] = -__builtin_inff();
      b[j] = -1;
    }
  }

  __device__ __forceinline__ void offer(float x, int blk) {
    if (x > v[L - 1]) {
      // position p = #{j : v[j] >= x}; entries from p move down by one.
#pragma unroll
      for (int j = L - 1; j >= 1; --j) {
        const bool keep = v[j] >= x;
        const bool prev = v[j - 1] >= x;
        const float nv = keep ? v[j] : (prev ? x : v[j - 1]);
        const int nb = keep ? b[j] : (prev ? blk : b[j - 1]);
        v[j] = nv;
        b[j] = nb;
      }
      if (!(v[0] >= x)) {
        v[0] = x;
        b[0] = blk;
      }
    }
  }

  // Remove the head (used when merging lists across lanes).
  __device__ __forceinline__ void pop() {
#pragma unroll
    for (int j = 0; j < L - 1; ++j) {
      v[j] = v[j + 1];
      b[j] = b[j + 1];
    }
    v[L - 1] = -__builtin_inff();
    b[L - 1] = -1;
  }
};

// 32-bit selection key of a finite block score: the score's order-preserving
// unsigned image with its low bits (imask = 2^ib - 1, ib bits to number the blocks)
// replaced by imask - block.  A larger key is a better block: a higher score first,
// and among scores whose images agree above the low ib bits, the lower block.  The
// rounding keeps 23 - ib mantissa bits (relative resolution 2^-(23-ib)); -0.0 is
// taken as +0.0.  Key 0 is below every real key and means "no block".
__device__ __forceinline__ uint32_t block_key(float v, int blk, uint32_t imask) {
  uint32_t u = __float_as_uint(v);
  u = u == 0x80000000u ? 0u : u;
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (ord & ~imask) | (imask - (uint32_t)blk);
}

__device__ __forceinline__ int block_key_block(uint32_t key, uint32_t imask) {
  return key == 0u ? -1 : (int)(imask - (key & imask));
}

__device__ __forceinline__ uint32_t med3_u32(uint32_t a, uint32_t b, uint32_t c) {
  uint32_t r;
  asm("v_med3_u32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Top-L list of distinct 32-bit keys kept in registers by one lane, descending.
// Inserting x: position j takes the median of (old k[j-1], x, old k[j]), which is
// k[j-1] when x lies above it, x when x falls between, k[j] otherwise; so one
// branchless instruction per position, and offering 0 (or anything below k[L-1])
// changes nothing.
template <int L>
struct KeyList {
  uint32_t k[L];

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int j = 0; j < L; ++j) k[j] = 0u;
  }

  __device__ __forceinline__ void offer(uint32_t x) {
#pragma unroll
    for (int j = L - 1; j >= 1; --j) k[j] = med3_u32(k[j - 1], x, k[j]);
    k[0] = k[0] > x ? k[0] : x;
  }
};

// Wave-wide maximum of a 64-bit key, returned to every lane, with DPP lane moves
// (register-speed) instead of LDS shuffles: quad xor 1 and xor 2, half-row and row
// mirrors, then the row broadcasts 15 and 31 leave the maximum in lane 63.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t x) {
  const int lo = (int)(uint32_t)x, hi = (int)(uint32_t)(x >> 32);
  const uint32_t nlo = (uint32_t)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xf, false);
  const uint32_t nhi = (uint32_t)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xf, false);
  return ((uint64_t)nhi << 32) | nlo;
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  x = max_u64(x, dpp_u64<0xB1, 0xf>(x));   // quad_perm [1,0,3,2]
  x = max_u64(x, dpp_u64<0x4E, 0xf>(x));   // quad_perm [2,3,0,1]
  x = max_u64(x, dpp_u64<0x141, 0xf>(x));  // row_half_mirror
  x = max_u64(x, dpp_u64<0x140, 0xf>(x));  // row_mirror
  x = max_u64(x, dpp_u64<0x142, 0xa>(x));  // row_bcast:15 into rows 1 and 3
  x = max_u64(x, dpp_u64<0x143, 0xc>(x));  // row_bcast:31 into rows 2 and 3
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// (value, block) packed so that a larger key means a better entry: value
// descending, then block ascending; empty entries (block < 0) get key 0.  -0.0 is
// taken as +0.0 first, so the two zeros tie (lower block first) as they compare
// equal in the float comparisons of TopList.
__device__ __forceinline__ uint64_t rank_key(float v, int blk) {
  uint32_t u = __float_as_uint(v);
  u = u == 0x80000000u ? 0u : u;
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return blk < 0 ? 0ull : ((uint64_t)ord << 32) | (uint32_t)(0x7fffffff - blk);
}

__device__ __forceinline__ int rank_key_block(uint64_t key) {
  return key == 0ull ? -1 : 0x7fffffff - (int)(uint32_t)key;
}

// Merge two descending runs a[0..N/2) and a[N/2..N) (the second stored reversed,
// i.e. ascending) into one descending run: the bitonic merge network.
template <int N>
__device__ __forceinline__ void bitonic_merge_desc(uint64_t (&a)[N]) {
#pragma unroll
  for (int stride = N >> 1; stride > 0; stride >>= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int j = i ^ stride;
      if (j > i) {
        const uint64_t x = a[i], y = a[j];
        const bool sw = y > x;
        a[i] = sw ? y : x;
        a[j] = sw ? x : y;
      }
    }
  }
}

template <int N>
__device__ __forceinline__ void bitonic_merge_desc(uint32_t (&a)[N]) {
#pragma unroll
  for (int stride = N >> 1; stride > 0; stride >>= 1) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int j = i ^ stride;
      if (j > i) {
        const uint32_t x = a[i], y = a[j];
        a[i] = x > y ? x : y;
        a[j] = x > y ? y : x;
      }
    }
  }
}

template <int N>
__device__ __forceinline__ void bitonic_sort_asc(int (&a)[N]) {
#pragma unroll
  for (int size = 2; size <= N; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int j = i ^ stride;
        if (j > i) {
          const bool asc = (i & size) == 0;
          const int x = a[i], y = a[j];
          const int lo = x < y ? x : y, hi = x < y ? y : x;
          a[i] = asc ? lo : hi;
          a[j] = asc ? hi : lo;
        }
      }
    }
  }
}

// Final selection for one (query, group): the first k-1 kept blocks plus the local
// block b_loc, ascending, then -1 padding.  `cand` holds N >= k entries, with
// INT_MAX for "no block".  Writes k ints to out.
template <int N>
__device__ __forceinline__ void write_selection(int (&cand)[N], int k, int b_loc, int32_t* out) {
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < N; ++j) cnt += cand[j] != 0x7fffffff;
  bitonic_sort_asc<N>(cand);
#pragma unroll
  for (int t = 0; t < N; ++t) {
    if (t < k) out[t] = t < cnt ? cand[t] : (t == cnt ? b_loc : -1);
  }
}

// Dynamic item schedule of the persistent-grid kernels (the pages balance their
// variable work with a persistent grid and a global atomic counter).  Workgroup w runs
// on XCD w % 8.  The items of XCD x are, in order, items
//   (t / per) * grid + x * per + t % per,   t = 0, 1, ...   (per = grid / 8),
// runs of `per` consecutive items, mostly of one list, so that a staged K/V block is
// re-read from that XCD's L2.  Each XCD hands its items out through its own counter
// (ctr[x * stride], zeroed before the launch); a workgroup whose XCD has none left
// takes the next XCD's, and so on, and stops when all eight are exhausted.  Only one
// thread of a workgroup uses the queue.  take() issues the atomic for a ticket;
// resolve() turns it into an item (or -1), taking more tickets past an exhausted XCD.
struct ItemQueue {
  int32_t* ctr;
  int64_t n_items;
  int grid, per, xcd, stride, off;
  __device__ int take() { return atomicAdd(ctr + ((xcd + off) & 7) * stride, 1); }
  __device__ int64_t resolve(int t) {
    for (;;) {
      const int x = (xcd + off) & 7;
      const int64_t item = (int64_t)(t / per) * grid + (int64_t)x * per + t % per;
      if (item < n_items) return item;
      if (++off == 8) return -1;
      t = take();
    }
  }
};

// Stores the next item into the workgroup's LDS slot and waits until the store has
// completed (lgkmcnt(0); vmcnt and expcnt left alone), so that a barrier that follows
// publishes it to every wave.
__device__ __forceinline__ void publish_item(int64_t* slot, int64_t item) {
  *slot = item;
  __builtin_amdgcn_s_waitcnt(0xC07F);
}

// Load-balance measurement of the persistent-grid kernels: with clk set, thread 0 of
// every workgroup stores the constant-rate (100 MHz) clock at its start (slot 0) and,
// after its last item, at its end (slot 1), in clk[2 * blockIdx.x + slot].  clk is a
// kernel argument (uniform), so the check costs nothing when it is null.
__device__ __forceinline__ void wg_clock_start(uint64_t* clk) {
  if (clk && threadIdx.x == 0) clk[2 * blockIdx.x] = __builtin_amdgcn_s_memrealtime();
}
__device__ __forceinline__ void wg_clock_end(uint64_t* clk) {
  if (clk) {
    __syncthreads();
    if (threadIdx.x == 0) clk[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime();
  }
}

// ---------------------------------------------------------------------------------
// K / V block staging shared by the prefill and decode attention kernels (256
// threads).
// LDS row rho of the staged K tile holds key swap23(rho) (bits 2 and 3 of the row
// index exchanged).  With that order the 32x32 MFMA leaves, in each lane half, the
// probabilities of 8 consecutive keys per PV step, so V^T is read 16 B at a time.
__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// 16-byte load, optionally non-temporal (data read once).
template <bool NT>
__device__ __forceinline__ u32x4_t ld16(const uint16_t* p) {
  if constexpr (NT)
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  else
    return *reinterpret_cast<const u32x4_t*>(p);
}

// K block -> LDS: row rho (256 B = 16 chunks of 16 B) holds key swap23(rho), chunk c
// at position c ^ (rho & 15).  kb points at (the block's first token, group r); all
// 128 rows past `nvalid` read as zero (a 64-key block fills half the tile).
template <bool NT = false>
__device__ __forceinline__ void stage_k(const uint16_t* __restrict__ kb, int row_stride, int nvalid, uint8_t* Ks,
                                        int tid) {
  const int c = tid & 15;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int rho = (tid >> 4) + 16 * m;
    const int key = swap23(rho);
    const int kr = key < nvalid ? key : nvalid - 1;  // branch-free: clamp, then zero
    u32x4_t val = ld16<NT>(kb + kr * row_stride + c * 8);
    if (key >= nvalid) val = u32x4_t{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4_t*>(Ks + rho * 256 + ((c ^ (rho & 15)) << 4)) = val;
  }
}

// V block -> LDS transposed: Vt[d] (256 B) holds keys in natural order, 8-key chunk
// kc at position kc ^ (d & 15).  vb points at (the block's first token, group r);
// keys past `nvalid` read as zero.
template <bool NT = false>
__device__ __forceinline__ void stage_v(const uint16_t* __restrict__ vb, int row_stride, int nvalid, uint8_t* Vt,
                                        int tid) {
  // Thread owns keys kg*8 .. +7 x dims dc*8 .. +7, transposed in registers.
  const int kg = tid & 15;
  const int dc = tid >> 4;
  uint32_t w[8][4];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int key = kg * 8 + e;
    const int kr = key < nvalid ? key : nvalid - 1;
    u32x4_t val = ld16<NT>(vb + kr * row_stride + dc * 8);
    if (key >= nvalid) val = u32x4_t{0u, 0u, 0u, 0u};
    w[e][0] = val.x;
    w[e][1] = val.y;
    w[e][2] = val.z;
    w[e][3] = val.w;
  }
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    // dim d = dc*8+f for keys kg*8 .. +7: 4 dwords of (key 2m, key 2m+1)
    u32x4_t o4;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t a = w[2 * m][f >> 1], cc = w[2 * m + 1][f >> 1];
      o4[m] = (f & 1) ? ((a >> 16) | (cc & 0xffff0000u)) : ((a & 0xffffu) | (cc << 16));
    }
    const int d = dc * 8 + f;
    *reinterpret_cast<u32x4_t*>(Vt + d * 256 + ((kg ^ (d & 15)) << 4)) = o4;
  }
}

__device__ __forceinline__ void stage_kv(const uint16_t* __restrict__ kb, const uint16_t* __restrict__ vb,
                                         int row_stride, int nvalid, uint8_t* Ks, uint8_t* Vt, int tid) {
  stage_k(kb, row_stride, nvalid, Ks, tid);
  stage_v(vb, row_stride, nvalid, Vt, tid);
}

}  // namespace msa
