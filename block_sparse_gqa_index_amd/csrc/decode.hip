// Decode kernels: one new token per sequence against packed variable-length caches.
//
// Method: the same Index Branch and Main Branch (page "MiniMax Sparse Attention
// (MSA)" paper review, section 3, Eq. 6-8) for the single query at position
// L_s - 1 of each sequence, whose local block is the last cache block; the pages
// report a decode speed-up from the same selection (paper review, result 3) and
// the open interface has a decode path over a KV cache (reading notes, 5.4).
//
// Four launches, all bandwidth-bound:
//   1. score: the index keys of every cached token are streamed once (128 B per
//      token); 16x16x32 MFMAs give all groups' scores, max-pooled per block.
//   2. top-k: one wave per (sequence, group); per-lane register lists over a
//      strided share of the blocks, merged by k-1 rounds of wave arg-max.
//   3. split-K attention: one workgroup per (sequence, group, part of up to 8
//      chosen blocks) streams those blocks' K/V (64 KB each) once for the G heads
//      of the group, with an online softmax across the part's blocks.
//   4. combine: LSE merge of the parts per (sequence, head).
#include <type_traits>

#include "msa_device.h"
#include "msa_kernels.h"
#include "table_clamp.h"

namespace msa {

namespace {

constexpr int kScoreBlocksPerWG = 4;  // one block (128 keys) per wave

// Where a sequence's cached tokens live.  The caller's tables (offsets, lengths, page
// numbers) are read through the clamps of table_clamp.h, so that a malformed table
// cannot move an access outside the cache buffers; every kernel reads a sequence's
// tokens 0 .. len(s) - 1 only.
// Packed: sequences back to back (offsets cu), bf16 K/V rows [T][H_kv][d_h].
// BK: keys per block (64 or 128), a compile-time constant so that the block
// arithmetic stays shifts.
template <int BK>
struct PackedCache {
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* kidx;
  const int64_t* cu;
  int64_t T;  // cached tokens (rows of k, v and kidx)
  static constexpr int bk = BK;
  __device__ int64_t start(int s) const { return clamp_i64(cu[s], 0, T); }
  __device__ int64_t len(int s) const { return packed_span(cu[s], cu[s + 1], T).len; }
  // Index key 64h of 128-key tile t of sequence s (keys are consecutive rows).
  __device__ const uint16_t* kidx_half(int s, int64_t t, int h, int64_t) const {
    return kidx + (start(s) + t * kBk + 64 * h) * kDidx;
  }
  // Element offset of (block b, key 0, group r) in the K/V rows; rows are H_kv * d_h apart.
  __device__ int64_t kv_block(int s, int64_t b, int r, int H_kv) const {
    return ((start(s) + b * bk) * H_kv + r) * kDh;
  }
};

// Paged: pages of BK tokens (one block), token j of sequence s in row j % BK of
// page table[s][j / BK]; K/V pages hold FP8 E4M3 codes (K = k_scale * value, V =
// v_scale * value, the scales applied by the caller's arithmetic), index-key pages bf16.
template <int BK>
struct PagedFp8Cache {
  const uint8_t* k;
  const uint8_t* v;
  const uint16_t* kidx;
  const int32_t* table;
  int64_t max_blocks;
  const int64_t* lens;
  int64_t num_pages;  // pages in k, v and kidx
  static constexpr int bk = BK;
  // At most max_blocks pages, so every table entry read is in its row.
  __device__ int64_t len(int s) const { return paged_len(lens[s], max_blocks, BK); }
  __device__ int64_t page(int s, int64_t b) const {
    return page_number(table[(int64_t)s * max_blocks + b], num_pages);
  }
  // Index key 64h of 128-key tile t.  With 64-token pages the half is a page of its
  // own; a half past the sequence end (L tokens) reads no table entry of it.
  __device__ const uint16_t* kidx_half(int s, int64_t t, int h, int64_t L) const {
    if constexpr (BK == 64) {
      const int64_t last = (L - 1) / BK;
      const int64_t pb = (2 * t + h < last) ? 2 * t + h : last;
      return kidx + page(s, pb) * BK * kDidx;
    } else {
      return kidx + (page(s, t) * BK + 64 * h) * kDidx;
    }
  }
  __device__ int64_t kv_block(int s, int64_t b, int r, int H_kv) const {
    return (page(s, b) * BK * H_kv + r) * kDh;
  }
};

// Eight FP8 E4M3 codes -> eight bf16 (exact: an E4M3 value has at most 4
// significant bits, so its f32 form has zero low halves).
__device__ __forceinline__ u32x4_t fp8x8_to_bf16x8(u32x2_t w) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
  const f2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
  const f2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
  const f2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
  auto pk = [](float lo, float hi) { return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u); };
  return u32x4_t{pk(a.x, a.y), pk(b.x, b.y), pk(c.x, c.y), pk(d.x, d.y)};
}

template <class Cache>
__global__ __launch_bounds__(256) void dec_score_kernel(const uint16_t* __restrict__ q_idx, Cache cache, int H_kv,
                                                        int64_t Bmax, float* __restrict__ M) {
  __shared__ __attribute__((aligned(16))) uint8_t kstage[kScoreBlocksPerWG][64 * 128];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int s = blockIdx.x;
  const int64_t L = cache.len(s);
  const int bk = cache.bk;
  const int64_t nb = (L + kBk - 1) / kBk;  // 128-key tiles of this sequence
  const int64_t b = (int64_t)blockIdx.y * kScoreBlocksPerWG + wave;
  if (b >= nb || b * (kBk / bk) >= Bmax) return;
  const uint16_t* __restrict__ kb0 = cache.kidx_half(s, b, 0, L);
  const uint16_t* __restrict__ kb1 = cache.kidx_half(s, b, 1, L);
  const int col = lane & 15, grp = lane >> 4;
  uint4 qop[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    qop[ks] = col < H_kv ? *reinterpret_cast<const uint4*>(q_idx + ((int64_t)s * H_kv + col) * kDidx + ks * 32 + 8 * grp)
                         : make_uint4(0, 0, 0, 0);
  // The block's 128 index keys (16 KB, read once per step: non-temporal) are all
  // requested before the first MFMA, fully coalesced: load j of lane l reads
  // 16-byte chunk l%8 of row 8j + l/8.  Keys past the sequence end re-read its last
  // key (a valid address); their scores are masked below.  Rows 64 and up of the tile
  // come from its second half (for j < 8 the row is below 64 by construction).
  u32x4_t raw[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int64_t key = b * kBk + 8 * j + (lane >> 3);
    const int kr = (int)((key < L ? key : L - 1) - b * kBk);
    const uint16_t* row = (j < 8 || kr < 64) ? kb0 + kr * kDidx : kb1 + (kr - 64) * kDidx;
    raw[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(row + (lane & 7) * 8));
  }
  // Half a block at a time through the wave's LDS buffer into the MFMA operand
  // layout (lane (col, grp) holds row col of a 16-row tile, dims 32ks + 8grp ..
  // +7): row rr of the half at rr*128, chunk c at position c ^ (rr & 7).
  uint8_t* st = kstage[wave];
  float hmax[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    float runmax = -__builtin_inff();
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int rr = 8 * jj + (lane >> 3);
      *reinterpret_cast<u32x4_t*>(st + rr * 128 + (((lane & 7) ^ (rr & 7)) << 4)) = raw[8 * hf + jj];
    }
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int rr = 16 * kt + col;
      f32x4_t acc = {};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int c = 4 * ks + grp;
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(st + rr * 128 + ((c ^ (rr & 7)) << 4));
        acc = mfma_16x16x32(as_bf16x8(a), as_bf16x8(qop[ks]), acc);
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t pos = b * kBk + 64 * hf + kt * 16 + 4 * grp + v;
        runmax = fmaxf(runmax, pos < L ? acc[v] : -__builtin_inff());
      }
    }
    runmax = fmaxf(runmax, __shfl_xor(runmax, 16));
    hmax[hf] = fmaxf(runmax, __shfl_xor(runmax, 32));
  }
  // A 128-key tile is one block (B_k = 128) or blocks 2b and 2b+1 (B_k = 64).
  if (lane < 16 && col < H_kv) {
    float* mrow = M + ((int64_t)s * H_kv + col) * Bmax;
    if (bk == kBk) {
      mrow[b] = fmaxf(hmax[0], hmax[1]) * 0.125f;
    } else {
      const int64_t nblk = (L + bk - 1) / bk;
      mrow[2 * b] = hmax[0] * 0.125f;
      if (2 * b + 1 < nblk && 2 * b + 1 < Bmax) mrow[2 * b + 1] = hmax[1] * 0.125f;
    }
  }
}

// Top-k of one (sequence, group) row per workgroup: wave w offers blocks
// 64j + lane with (j % 4) == w to per-lane register lists, extracts its k-1 best
// by k-1 rounds of wave arg-max, and the four waves' candidates are merged by
// wave 0 the same way.  The local (last) block is then added.
template <int LIST, class Cache>
__global__ __launch_bounds__(256) void dec_topk_kernel(const float* __restrict__ M, Cache cache, int batch, int H_kv,
                                                       int64_t Bmax, int k, int32_t* __restrict__ block_idx) {
  __shared__ uint64_t cand[4][LIST];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.x;
  const int s = (int)(row / H_kv);
  const int64_t L = cache.len(s);
  int32_t* out = block_idx + row * k;
  if (L <= 0) {
    for (int t = threadIdx.x; t < k; t += 256) out[t] = -1;
    return;
  }
  int64_t bl = (L - 1) / cache.bk;
  if (bl > Bmax - 1) bl = Bmax - 1;
  TopList<LIST> list;
  list.init();
  const float* mrow = M + row * Bmax;
  // Scores are loaded in batches of 8 per lane before any is offered.
  for (int64_t b0 = 64 * wave; b0 < bl; b0 += 8 * 256) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t b = b0 + lane + 256 * j;
      v[j] = mrow[b < bl ? b : 0];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t b = b0 + lane + 256 * j;
      if (b < bl) list.offer(v[j], (int)b);
    }
  }
  // This wave's k-1 best, best first.
#pragma unroll
  for (int t = 0; t < LIST; ++t) {
    uint64_t best = 0;
    if (t < k - 1) {
      const uint64_t mine = rank_key(list.v[0], list.b[0]);
      best = wave_max_u64(mine);
      if (best != 0 && mine == best) list.pop();
    }
    if (lane == 0) cand[wave][t] = best;
  }
  __syncthreads();
  if (wave != 0) return;
  // Merge: candidate c = LIST*w + t (wave w's t-th) sits in lane c % 64, slot c / 64
  // (at most 4*31 = 124 candidates); the waves' blocks are disjoint.
  const uint64_t* flat = &cand[0][0];
  const uint64_t c0 = lane < 4 * LIST ? flat[lane] : 0, c1 = lane + 64 < 4 * LIST ? flat[lane + 64] : 0;
  uint64_t hi = c0 > c1 ? c0 : c1, lo = c0 > c1 ? c1 : c0;
  int sel[LIST + 1];
#pragma unroll
  for (int t = 0; t <= LIST; ++t) sel[t] = 0x7fffffff;
#pragma unroll
  for (int t = 0; t < LIST; ++t) {
    if (t < k - 1) {
      const uint64_t best = wave_max_u64(hi);
      if (best != 0) {
        sel[t] = rank_key_block(best);
        if (hi == best) {
          hi = lo;
          lo = 0;
        }
      }
    }
  }
  if (lane == 0) {
    int32_t o[LIST + 1];
    write_selection<LIST + 1>(sel, k, (int)bl, o);
#pragma unroll
    for (int t = 0; t <= LIST; ++t)
      if (t < k) out[t] = o[t];
  }
}

// Split-K attention: one workgroup per (sequence, group, part), a part being up
// to kDecSlotsPerPart of the row's selected blocks; parts are merged by the
// combine kernel.  The G heads of the group are the (32, G real) MFMA columns of
// 32x32x16 bf16 MFMAs.  The workgroup stages each block's K and V rows in LDS from
// coalesced loads (V^T operands are then read with transposing LDS reads); while a
// block is computed the next block's K and V are already being loaded into
// registers.  Wave w takes keys
// 32w .. 32w+31 of every block (S^T = K Q^T), keeps a running max, sum and output
// over the part's blocks (online softmax, base 2) and computes O^T = V^T P^T.  At the end the four waves' (max, sum, O) are merged in LDS
// (rescaled to the common max) and the normalised partial with its natural-log
// LSE is written (LSE -inf: the part attended to nothing).
constexpr int kDecSlotsPerPart = 8;

// FP8 caches: the codes are widened to bf16 (exactly) on their way to LDS; the K
// scale is folded into scale_log2 and the V scale (v_mul) into the partial output.
template <int G, class Cache>
__global__ __launch_bounds__(256, 2) void dec_attn_kernel(const uint16_t* __restrict__ q, Cache cache,
                                                          const int32_t* __restrict__ block_idx, int H_kv,
                                                          int kk, int nparts, float scale_log2, float v_mul,
                                                          float* __restrict__ Opart, float* __restrict__ Lpart) {
  constexpr bool kFp8 = sizeof(*cache.k) == 1;
  static_assert(G <= 16, "the merge reuses the 32 KB V buffer: 4 x G x 128 fp32");
  __shared__ __attribute__((aligned(16))) uint8_t Ks[kBk * 256];
  __shared__ __attribute__((aligned(16))) uint8_t Vs[kBk * 256];  // V rows; reused for the merge
  __shared__ float wm[4][32], wl[4][32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t task = blockIdx.x;  // (s * H_kv + r) * nparts + part
  const int64_t sr = task / nparts;
  const int part = (int)(task % nparts);
  const int s = (int)(sr / H_kv), r = (int)(sr % H_kv);
  const int64_t L = cache.len(s);
  const int H_q = H_kv * G;
  const int row_stride = H_kv * kDh;  // elements between a group's consecutive key rows
  const int32_t* sel = block_idx + sr * kk;
  const int t0 = part * kDecSlotsPerPart;
  const int t1 = (t0 + kDecSlotsPerPart < kk) ? t0 + kDecSlotsPerPart : kk;
  const int bk = cache.bk;
  const int64_t bl = L > 0 ? (L - 1) / bk : -1;
  // Next selected, valid slot at or after t (t1 if none); uniform.
  auto next_valid = [&](int t) {
    while (t < t1 && !(sel[t] >= 0 && sel[t] <= bl)) ++t;
    return t;
  };
  int t = next_valid(t0);
  float* lp = Lpart + task * G;
  if (t >= t1) {
    if (tid < G) lp[tid] = -__builtin_inff();
    return;
  }
  // Loads of one block into registers, coalesced: K as 8 rows x 8 dims per thread
  // (row (tid >> 4) + 16m holds key swap23 of it, dims 8 * (tid & 15) ..), V as 8
  // keys x 8 dims per thread; keys past the end are clamped, then zeroed.  FP8 rows
  // arrive as 8-byte pieces and are widened in store_block.  Both are read once, with
  // non-temporal loads (K too: 272 against 278-284 us for the 64 x 128K step).
  using Raw = typename std::conditional<kFp8, u32x2_t, u32x4_t>::type;
  Raw kr[8], vr[8];
  auto load8 = [&](const auto* p, bool nt) -> Raw {
    if constexpr (kFp8)
      return nt ? __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p))
                : *reinterpret_cast<const u32x2_t*>(p);
    else
      return nt ? ld16<true>(p) : ld16<false>(p);
  };
  auto load_block = [&](int b) {
    const int64_t kb0 = (int64_t)b * bk;
    const int nvalid = (L - kb0 < bk) ? (int)(L - kb0) : bk;
    const int64_t base = cache.kv_block(s, b, r, H_kv);
    const int c = tid & 15;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int key = swap23((tid >> 4) + 16 * m);
      kr[m] = load8(cache.k + base + (int64_t)(key < nvalid ? key : nvalid - 1) * row_stride + c * 8, true);
      if (key >= nvalid) kr[m] = Raw{};
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int key = (tid >> 4) + 16 * m;
      vr[m] = load8(cache.v + base + (int64_t)(key < nvalid ? key : nvalid - 1) * row_stride + c * 8, true);
      if (key >= nvalid) vr[m] = Raw{};
    }
  };
  auto widen = [&](const Raw& x) -> u32x4_t {
    if constexpr (kFp8)
      return fp8x8_to_bf16x8(x);
    else
      return x;
  };
  // The block to LDS from the registers: K row rho (256 B) at rho*256 and V row key
  // at key*256, chunk c at position c ^ (row & 15).
  auto store_block = [&]() {
    const int c = tid & 15;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const int rho = (tid >> 4) + 16 * m;
      *reinterpret_cast<u32x4_t*>(Ks + rho * 256 + ((c ^ (rho & 15)) << 4)) = widen(kr[m]);
      *reinterpret_cast<u32x4_t*>(Vs + rho * 256 + ((c ^ (rho & 15)) << 4)) = widen(vr[m]);
    }
  };
  // q operand: k-slot (h, e) of step st is dim 64h + 8st + e of head l32 (zero for
  // the padding columns l32 >= G).
  u32x4_t qop[8];
  {
    const uint16_t* qr = q + ((int64_t)s * H_q + r * G + (l32 < G ? l32 : 0)) * kDh + 64 * h;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(qr + 8 * st);
      qop[st] = l32 < G ? v : u32x4_t{0u, 0u, 0u, 0u};
    }
  }
  int b = sel[t];
  load_block(b);
  store_block();
  float m_run = -__builtin_inff(), l_run = 0.f;  // base-2 scaled max, sum (per column)
  f32x16_t oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16_t{};
  while (true) {
    const int64_t kb0 = (int64_t)b * bk;
    const int nvalid = (L - kb0 < bk) ? (int)(L - kb0) : bk;
    const int tn = next_valid(t + 1);
    const int bn = tn < t1 ? sel[tn] : b;
    __syncthreads();  // this block's K and V^T staged
    // The staging registers are free: the next block's loads go in flight while
    // this block is computed.
    if (tn < t1) load_block(bn);

    // S^T tile of this wave (LDS row 32w + l32 holds key 32w + swap23(l32)):
    // element v is key 32w + 16(v/8) + 4((v/4)%2) + v%4 + 8h.
    f32x16_t sacc = f32x16_t{};
    {
      const int row = 32 * wave + l32;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const int c = 8 * h + st;
        const u32x4_t a = *reinterpret_cast<const u32x4_t*>(Ks + row * 256 + ((c ^ (row & 15)) << 4));
        sacc = mfma_32x32x16(as_bf16x8(a), as_bf16x8(qop[st]), sacc);
      }
    }
    if (nvalid < kBk) {
      const int lim = nvalid - 1 - 32 * wave - 8 * h;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int off = 16 * (v >> 3) + 4 * ((v >> 2) & 1) + (v & 3);
        sacc[v] = off <= lim ? sacc[v] : -__builtin_inff();
      }
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, sacc[v]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx == -__builtin_inff() ? -__builtin_inff() : mx * scale_log2);
    // Rescale what was accumulated so far (nothing to rescale while m_run = -inf).
    const float alpha = m_run == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
    const float msub = m_new == -__builtin_inff() ? 0.f : m_new;
    float lt = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sacc[v], scale_log2, -msub));
      sacc[v] = p;
      lt += p;
    }
    lt += __shfl_xor(lt, 32);
    l_run = l_run * alpha + lt;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;
    }
    u32x4_t pb[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      pb[hf].x = pack_bf16x2(sacc[8 * hf + 0], sacc[8 * hf + 1]);
      pb[hf].y = pack_bf16x2(sacc[8 * hf + 2], sacc[8 * hf + 3]);
      pb[hf].z = pack_bf16x2(sacc[8 * hf + 4], sacc[8 * hf + 5]);
      pb[hf].w = pack_bf16x2(sacc[8 * hf + 6], sacc[8 * hf + 7]);
    }
    // O^T[d][head] += V^T P^T over this wave's keys: step u = 2w + hf takes keys
    // 8(2u + h) .. +7 for lane half h.  The V^T operand (8 keys of one dim per lane)
    // comes from the V rows by transposing LDS reads: within each group of 16 lanes,
    // lane i receives element i % 4 of the 8 bytes read by lane 4k + i / 4 (k = 0..3),
    // so lane j reads dims 4(j % 4) .. +3 of key K0 + j / 4 and lane i gets keys
    // K0 .. K0+3 of dim i.
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int K0 = 8 * (2 * (2 * wave + hf) + h);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int d0 = dt * 32 + (l32 & 16);  // this lane group's 16 dims
        u32x2_t half[2];
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          const int key = K0 + 4 * part + ((lane & 15) >> 2);
          const int col = d0 + 4 * (lane & 3);
          const uint8_t* p = Vs + key * 256 + ((((col >> 3) ^ (key & 15))) << 4) + (col & 7) * 2;
          typedef short v4i16 __attribute__((ext_vector_type(4)));
          half[part] = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                       (v4i16 __attribute__((address_space(3)))*)(const_cast<uint8_t*>(p))));
        }
        const u32x4_t va = u32x4_t{half[0][0], half[0][1], half[1][0], half[1][1]};
        oacc[dt] = mfma_32x32x16(as_bf16x8(va), as_bf16x8(pb[hf]), oacc[dt]);
      }
    }
    __syncthreads();  // every wave is done with this block's K and V^T
    if (tn >= t1) break;
    store_block();
    t = tn;
    b = bn;
  }
  if (h == 0) {
    wm[wave][l32] = m_run;
    wl[wave][l32] = l_run;
  }
  // Merge: the four waves' O^T for the G real heads, rescaled to the common max.
  float* red = reinterpret_cast<float*>(Vs);  // [4][G][128]
  if (l32 < G) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int d = 32 * dt + 8 * c + 4 * h;
        *reinterpret_cast<f32x4_t*>(red + ((wave * G + l32) * kDh + d)) =
            f32x4_t{oacc[dt][4 * c], oacc[dt][4 * c + 1], oacc[dt][4 * c + 2], oacc[dt][4 * c + 3]};
      }
    }
  }
  __syncthreads();
  float* op = Opart + task * G * kDh;
  for (int e = tid; e < G * kDh; e += 256) {
    const int g = e / kDh, d = e % kDh;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w][g]);
    float acc = 0.f, ls = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float wt = wm[w][g] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(wm[w][g] - M);
      acc += wt * red[(w * G + g) * kDh + d];
      ls += wt * wl[w][g];
    }
    op[e] = acc / ls * v_mul;
    if (d == 0) lp[g] = (M + __log2f(ls)) * kLn2;
  }
}

// LSE merge of the parts of one (sequence, head) per wave: lane p < nparts reads
// part p's LSE (-inf: the part attended to nothing); the common max and each part's
// weight are wave reductions and lane reads; lane j then accumulates dims 2j, 2j+1.
__global__ __launch_bounds__(256) void dec_combine_kernel(const float* __restrict__ Opart,
                                                          const float* __restrict__ Lpart, int batch, int H_kv,
                                                          int G, int nparts, float* __restrict__ o,
                                                          float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int H_q = H_kv * G;
  if (gw >= (int64_t)batch * H_q) return;
  const int s = (int)(gw / H_q), hh = (int)(gw % H_q);
  const int r = hh / G, g = hh % G;
  const int64_t sr = (int64_t)s * H_kv + r;
  const float ls = lane < nparts ? Lpart[(sr * nparts + lane) * G + g] : -__builtin_inff();
  const bool valid = ls != -__builtin_inff();
  const float mstar = wave_max(ls);
  float* orow = o + gw * kDh;
  if (mstar == -__builtin_inff()) {
    *reinterpret_cast<float2*>(orow + 2 * lane) = make_float2(0.f, 0.f);
    if (lane == 0) lse[gw] = -__builtin_inff();
    return;
  }
  const float wgt = valid ? __expf(ls - mstar) : 0.f;
  const float Ls = wave_sum(wgt);
  const uint64_t vm = __ballot(valid);
  const int first = (int)__builtin_ctzll(vm);  // vm != 0 here
  float a0 = 0.f, a1 = 0.f;
  for (int u = 0; u < nparts; ++u) {
    const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), u));
    // Empty parts wrote no row: read the first non-empty part's row (weight 0).
    const int us = ((vm >> u) & 1) ? u : first;
    const float2 pv = *reinterpret_cast<const float2*>(Opart + ((sr * nparts + us) * G + g) * kDh + 2 * lane);
    a0 += wu * pv.x;
    a1 += wu * pv.y;
  }
  const float inv = 1.f / Ls;
  *reinterpret_cast<float2*>(orow + 2 * lane) = make_float2(a0 * inv, a1 * inv);
  if (lane == 0) lse[gw] = mstar + __logf(Ls);
}

}  // namespace

DecodeWorkspace decode_workspace_layout(int batch, int H_q, int H_kv, int kk, int64_t Bmax) {
  DecodeWorkspace L{};
  const int G = H_q / H_kv;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  L.M = take(sizeof(float) * (size_t)batch * H_kv * Bmax);
  const int nparts = (kk + kDecSlotsPerPart - 1) / kDecSlotsPerPart;
  L.opart = take(sizeof(float) * (size_t)batch * H_kv * nparts * G * kDh);
  L.lpart = take(sizeof(float) * (size_t)batch * H_kv * nparts * G);
  L.total = off;
  return L;
}

template <class Cache>
static hipError_t launch_decode_impl(const uint16_t* q, const uint16_t* q_idx, const Cache& cache, int batch,
                                     int64_t Bmax, int H_q, int H_kv, int kk, float scale_log2, float v_mul,
                                     int32_t* block_idx, float* o, float* lse, uint8_t* ws,
                                     const DecodeWorkspace& L, hipStream_t stream) {
  const int G = H_q / H_kv;
  float* M = reinterpret_cast<float*>(ws + L.M);
  float* opart = reinterpret_cast<float*>(ws + L.opart);
  float* lpart = reinterpret_cast<float*>(ws + L.lpart);
  hipError_t e;
  const int64_t tiles = (Bmax * cache.bk + kBk - 1) / kBk;  // 128-key tiles of the longest sequence
  dec_score_kernel<Cache><<<dim3((unsigned)batch, (unsigned)((tiles + kScoreBlocksPerWG - 1) / kScoreBlocksPerWG)),
                            dim3(256), 0, stream>>>(q_idx, cache, H_kv, Bmax, M);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const unsigned rows_grid = (unsigned)((int64_t)batch * H_kv);
  if (kk <= 8)
    dec_topk_kernel<7, Cache><<<dim3(rows_grid), dim3(256), 0, stream>>>(M, cache, batch, H_kv, Bmax, kk, block_idx);
  else if (kk <= 16)
    dec_topk_kernel<15, Cache><<<dim3(rows_grid), dim3(256), 0, stream>>>(M, cache, batch, H_kv, Bmax, kk, block_idx);
  else
    dec_topk_kernel<31, Cache><<<dim3(rows_grid), dim3(256), 0, stream>>>(M, cache, batch, H_kv, Bmax, kk, block_idx);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int nparts = (kk + kDecSlotsPerPart - 1) / kDecSlotsPerPart;
  const unsigned tasks = (unsigned)((int64_t)batch * H_kv * nparts);
  switch (G) {
#define MSA_DEC_CASE(GG)                                                                                   \
  case GG:                                                                                                 \
    dec_attn_kernel<GG, Cache><<<dim3(tasks), dim3(256), 0, stream>>>(q, cache, block_idx, H_kv, kk, nparts, \
                                                                      scale_log2, v_mul, opart, lpart);    \
    break;
    MSA_DEC_CASE(1)
    MSA_DEC_CASE(2)
    MSA_DEC_CASE(4)
    MSA_DEC_CASE(8)
    MSA_DEC_CASE(16)
#undef MSA_DEC_CASE
    default:
      return hipErrorInvalidValue;
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t waves = (int64_t)batch * H_q;
  dec_combine_kernel<<<dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream>>>(opart, lpart, batch, H_kv, G,
                                                                                  nparts, o, lse);
  return hipGetLastError();
}

hipError_t launch_decode(const uint16_t* q, const uint16_t* q_idx, const uint16_t* k_cache,
                         const uint16_t* v_cache, const uint16_t* k_idx_cache, const int64_t* cu, int batch,
                         int64_t T, int64_t Bmax, int bk, int H_q, int H_kv, int kk, float scale, int32_t* block_idx, float* o,
                         float* lse, uint8_t* ws, const DecodeWorkspace& L, hipStream_t stream) {
  if (bk == 64) {
    const PackedCache<64> cache{k_cache, v_cache, k_idx_cache, cu, T};
    return launch_decode_impl(q, q_idx, cache, batch, Bmax, H_q, H_kv, kk, scale * kLog2e, 1.f, block_idx, o, lse,
                              ws, L, stream);
  }
  const PackedCache<128> cache{k_cache, v_cache, k_idx_cache, cu, T};
  return launch_decode_impl(q, q_idx, cache, batch, Bmax, H_q, H_kv, kk, scale * kLog2e, 1.f, block_idx, o, lse, ws,
                            L, stream);
}

hipError_t launch_decode_paged(const uint16_t* q, const uint16_t* q_idx, const uint8_t* k_pages,
                               const uint8_t* v_pages, float k_scale, float v_scale, const uint16_t* kidx_pages,
                               const int32_t* block_table, int64_t max_blocks, int64_t num_pages,
                               const int64_t* seqlens, int batch, int64_t Bmax, int bk, int H_q, int H_kv, int kk, float scale, int32_t* block_idx,
                               float* o, float* lse, uint8_t* ws, const DecodeWorkspace& L, hipStream_t stream) {
  if (bk == 64) {
    const PagedFp8Cache<64> cache{k_pages, v_pages, kidx_pages, block_table, max_blocks, seqlens,
                                          num_pages};
    return launch_decode_impl(q, q_idx, cache, batch, Bmax, H_q, H_kv, kk, scale * k_scale * kLog2e, v_scale,
                              block_idx, o, lse, ws, L, stream);
  }
  const PagedFp8Cache<128> cache{k_pages, v_pages, kidx_pages, block_table, max_blocks, seqlens,
                                          num_pages};
  return launch_decode_impl(q, q_idx, cache, batch, Bmax, H_q, H_kv, kk, scale * k_scale * kLog2e, v_scale,
                            block_idx, o, lse, ws, L, stream);
}

}  // namespace msa
