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
// kItemChunks chunks; a chunk is 128 MFMA rows = (128 / G) gathered queries x G
// heads (query concatenation).  A workgroup stages the block's K (32 KB) and V^T
// (33 KB) in LDS once per item, then for each chunk every wave computes 32 rows:
// S^T = K * Q^T and O^T = V^T * P^T on 32x32x16 bf16 MFMAs, with the softmax in
// fp32 in between.  Every pair owns its partial slot [query][group][slot], so the
// partials of hot (sink) blocks spread over many workgroups without atomics.
#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {

namespace {

// --------------------------------------------------------------------- inverse index
// Pair validity: 0 <= b <= b_loc(i) and b < B.  Later blocks add no token.
__device__ __forceinline__ bool pair_valid(int b, int64_t i, int64_t B) {
  return b >= 0 && (int64_t)b < B && (int64_t)b <= i / kBk;
}

__global__ __launch_bounds__(256) void inv_count_kernel(const int32_t* __restrict__ block_idx, int64_t w0,
                                                        int64_t W, int H_kv, int kk, int64_t B, int TQ,
                                                        int32_t* __restrict__ counts) {
  extern __shared__ int32_t hist[];
  const int r = blockIdx.y;
  const int64_t q0 = w0 + (int64_t)blockIdx.x * TQ;
  const int64_t q1 = (q0 + TQ < w0 + W) ? q0 + TQ : w0 + W;
  const int64_t bmax = ((q1 - 1) / kBk < B - 1) ? (q1 - 1) / kBk : B - 1;
  for (int64_t b = threadIdx.x; b <= bmax; b += 256) hist[b] = 0;
  __syncthreads();
  const int64_t npairs = (q1 - q0) * kk;
  for (int64_t p = threadIdx.x; p < npairs; p += 256) {
    const int64_t i = q0 + p / kk;
    const int s = (int)(p % kk);
    const int b = block_idx[(i * H_kv + r) * kk + s];
    if (pair_valid(b, i, B)) atomicAdd(&hist[b], 1);
  }
  __syncthreads();
  for (int64_t b = threadIdx.x; b <= bmax; b += 256) {
    const int c = hist[b];
    if (c) atomicAdd(&counts[r * B + b], c);
  }
}

// One workgroup: exclusive scans of the per-list pair counts and item counts, the
// list offsets, the scatter cursors and the explicit item table.
__global__ __launch_bounds__(1024) void inv_scan_kernel(const int32_t* __restrict__ counts, int64_t L,
                                                        int item_q, int32_t* __restrict__ cursor,
                                                        int4* __restrict__ items, int32_t* __restrict__ n_items) {
  __shared__ int64_t sp[1024], si[1024];
  const int t = threadIdx.x;
  const int64_t per = (L + 1023) / 1024;
  const int64_t l0 = t * per, l1 = (l0 + per < L) ? l0 + per : L;
  int64_t ps = 0, is = 0;
  for (int64_t l = l0; l < l1; ++l) {
    const int c = counts[l];
    ps += c;
    is += (c + item_q - 1) / item_q;
  }
  sp[t] = ps;
  si[t] = is;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int64_t a = 0, bb = 0;
    if (t >= off) {
      a = sp[t - off];
      bb = si[t - off];
    }
    __syncthreads();
    sp[t] += a;
    si[t] += bb;
    __syncthreads();
  }
  int64_t poff = sp[t] - ps, ioff = si[t] - is;
  for (int64_t l = l0; l < l1; ++l) {
    const int c = counts[l];
    cursor[l] = (int32_t)poff;
    const int nit = (c + item_q - 1) / item_q;
    for (int it = 0; it < nit; ++it) {
      const int start = (int)poff + it * item_q;
      const int cnt = (c - it * item_q < item_q) ? c - it * item_q : item_q;
      items[ioff + it] = make_int4((int)l, start, cnt, 0);
    }
    poff += c;
    ioff += nit;
  }
  if (t == 1023) *n_items = (int32_t)si[1023];
}

template <int PPT>
__global__ __launch_bounds__(256) void inv_scatter_kernel(const int32_t* __restrict__ block_idx, int64_t w0,
                                                          int64_t W, int H_kv, int kk, int64_t B, int TQ,
                                                          int32_t* __restrict__ cursor,
                                                          int32_t* __restrict__ pairs) {
  extern __shared__ int32_t sh[];
  int32_t* hist = sh;
  int32_t* base = sh + B;
  const int r = blockIdx.y;
  const int64_t q0 = w0 + (int64_t)blockIdx.x * TQ;
  const int64_t q1 = (q0 + TQ < w0 + W) ? q0 + TQ : w0 + W;
  const int64_t bmax = ((q1 - 1) / kBk < B - 1) ? (q1 - 1) / kBk : B - 1;
  for (int64_t b = threadIdx.x; b <= bmax; b += 256) hist[b] = 0;
  __syncthreads();
  const int64_t npairs = (q1 - q0) * kk;
  int rank[PPT];
#pragma unroll
  for (int u = 0; u < PPT; ++u) {
    const int64_t p = threadIdx.x + 256 * u;
    rank[u] = -1;
    if (p < npairs) {
      const int64_t i = q0 + p / kk;
      const int s = (int)(p % kk);
      const int b = block_idx[(i * H_kv + r) * kk + s];
      if (pair_valid(b, i, B)) rank[u] = atomicAdd(&hist[b], 1);
    }
  }
  __syncthreads();
  for (int64_t b = threadIdx.x; b <= bmax; b += 256) {
    const int c = hist[b];
    if (c) base[b] = atomicAdd(&cursor[r * B + b], c);
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < PPT; ++u) {
    if (rank[u] < 0) continue;
    const int64_t p = threadIdx.x + 256 * u;
    const int64_t i = q0 + p / kk;
    const int s = (int)(p % kk);
    const int b = block_idx[(i * H_kv + r) * kk + s];
    pairs[base[b] + rank[u]] = (int32_t)(((i - w0) << 5) | s);
  }
}

// --------------------------------------------------------------------- phase 1
constexpr int kAttnThreads = 256;
constexpr int kVtStride = kBk * 2 + 8;  // bytes per d-row of V^T (padding spreads banks)

// K block -> LDS, row j (256 B = 16 chunks of 16 B), chunk c at position c ^ (j & 15).
// V block -> LDS transposed: Vt[d][key] with rows of kVtStride bytes.
// kb/vb point at (token b*128, group r); rows past `nvalid` read as zero.
__device__ __forceinline__ void stage_kv(const uint16_t* __restrict__ kb, const uint16_t* __restrict__ vb,
                                         int row_stride, int nvalid, uint8_t* Ks, uint8_t* Vt, int tid) {
  // K: 2048 chunks, 8 per thread (rows tid/16 + 16m, chunk tid%16).
  const int c = tid & 15;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const int key = (tid >> 4) + 16 * m;
    const int kr = key < nvalid ? key : nvalid - 1;  // branch-free: clamp, then zero
    uint4 val = *reinterpret_cast<const uint4*>(kb + kr * row_stride + c * 8);
    if (key >= nvalid) val = make_uint4(0, 0, 0, 0);
    *reinterpret_cast<uint4*>(Ks + key * 256 + ((c ^ (key & 15)) << 4)) = val;
  }
  // V: thread owns an 8-key x 8-dim tile, transposed in registers.
  const int dc = tid & 15;   // dims dc*8 .. +7
  const int kg = tid >> 4;   // keys kg*8 .. +7
  uint32_t w[8][4];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int key = kg * 8 + e;
    const int kr = key < nvalid ? key : nvalid - 1;
    uint4 val = *reinterpret_cast<const uint4*>(vb + kr * row_stride + dc * 8);
    if (key >= nvalid) val = make_uint4(0, 0, 0, 0);
    w[e][0] = val.x;
    w[e][1] = val.y;
    w[e][2] = val.z;
    w[e][3] = val.w;
  }
#pragma unroll
  for (int f = 0; f < 8; ++f) {
    // dim dc*8+f for keys kg*8 .. +7: 4 dwords of (key 2m, key 2m+1)
    uint32_t o4[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t a = w[2 * m][f >> 1], cc = w[2 * m + 1][f >> 1];
      o4[m] = (f & 1) ? ((a >> 16) | (cc & 0xffff0000u)) : ((a & 0xffffu) | (cc << 16));
    }
    uint8_t* dst = Vt + (dc * 8 + f) * kVtStride + kg * 16;
    *reinterpret_cast<uint2*>(dst) = make_uint2(o4[0], o4[1]);
    *reinterpret_cast<uint2*>(dst + 8) = make_uint2(o4[2], o4[3]);
  }
}

template <int G>
__global__ __launch_bounds__(kAttnThreads, 2) void attn_kvouter_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kp, const uint16_t* __restrict__ vp,
    const int4* __restrict__ items, const int32_t* __restrict__ n_items_ptr, const int32_t* __restrict__ pairs,
    int64_t N, int H_kv, int64_t B, int kk, int64_t w0, float scale_log2, uint16_t* __restrict__ Opart,
    float* __restrict__ Lpart) {
  constexpr int kQC = 128 / G;         // gathered queries per chunk
  __shared__ __attribute__((aligned(16))) uint8_t Ks[kBk * 256];
  __shared__ __attribute__((aligned(16))) uint8_t Vt[kDh * kVtStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int H_q = H_kv * G;
  const int n_items = *n_items_ptr;

  // Consecutive items (mostly of one list) go to the workgroups of one XCD, so the
  // staged K/V block is read from that XCD's L2.
  const int grid = gridDim.x;
  const int per_xcd = grid >> 3;
  const int xcd = blockIdx.x & 7, slot_in_xcd = blockIdx.x >> 3;
  for (int64_t round = 0;; ++round) {
    const int64_t item = round * grid + (int64_t)xcd * per_xcd + slot_in_xcd;
    if (item >= n_items) break;
    const int4 it = items[item];
    const int64_t r = it.x / B, b = it.x % B;
    const int start = it.y, cnt = it.z;

    __syncthreads();  // previous item's LDS reads are done
    {
      const int64_t tok0 = b * kBk;
      const int row_stride = H_kv * kDh;
      const int nvalid = (N - tok0 < kBk) ? (int)(N - tok0) : kBk;
      const int64_t base = tok0 * row_stride + r * kDh;
      stage_kv(kp + base, vp + base, row_stride, nvalid, Ks, Vt, tid);
    }
    __syncthreads();

    for (int cb = 0; cb < cnt; cb += kQC) {
      // Keep the LDS operand reads inside the chunk loop: hoisting them (they do
      // not change across chunks) would need 256 registers per lane.
      asm volatile("" ::: "memory");
      const int qrow = wave * 32 + l32;
      const int qs = qrow / G, g = qrow % G;
      const bool valid = cb + qs < cnt;
      // Rows past the end of the item re-read the item's first pair (a valid
      // address); their results are discarded.
      const int pr = pairs[start + (valid ? cb + qs : 0)];
      const int64_t i_local = pr >> 5;
      const int s = pr & 31;
      const int64_t i = w0 + i_local;

      uint4 qop[8];
      const uint16_t* qrow_p = q + (i * H_q + r * G + g) * kDh + 64 * h;
#pragma unroll
      for (int t = 0; t < 8; ++t) qop[t] = *reinterpret_cast<const uint4*>(qrow_p + 8 * t);

      // S^T[key][qrow]: k-slot (h, e) of step t is dim 64h + 8t + e in both operands.
      f32x16_t sacc[4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        sacc[kt] = f32x16_t{};
        const int key = kt * 32 + l32;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int c = 8 * h + t;
          const uint4 a = *reinterpret_cast<const uint4*>(Ks + key * 256 + ((c ^ (key & 15)) << 4));
          sacc[kt] = mfma_32x32x16(as_bf16x8(a), as_bf16x8(qop[t]), sacc[kt]);
        }
      }

      // Softmax over this block's keys, base-2 with the scale folded in.
      const bool need_mask = b * kBk + (kBk - 1) > i;
      float mx = -__builtin_inff();
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          float x = sacc[kt][v] * scale_log2;
          if (need_mask) {
            const int64_t j = b * kBk + kt * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
            x = j <= i ? x : -__builtin_inff();
          }
          sacc[kt][v] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool empty = mx == -__builtin_inff();
      float l = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = empty ? 0.f : exp2f(sacc[kt][v] - mx);
          sacc[kt][v] = p;
          l += p;
        }
      }
      l += __shfl_xor(l, 32);

      // P in bf16 as the B operand of step u (8 keys per lane half).
      uint4 pb[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int kt = u >> 1, hf = u & 1;
        pb[u].x = pack_bf16x2(sacc[kt][8 * hf + 0], sacc[kt][8 * hf + 1]);
        pb[u].y = pack_bf16x2(sacc[kt][8 * hf + 2], sacc[kt][8 * hf + 3]);
        pb[u].z = pack_bf16x2(sacc[kt][8 * hf + 4], sacc[kt][8 * hf + 5]);
        pb[u].w = pack_bf16x2(sacc[kt][8 * hf + 6], sacc[kt][8 * hf + 7]);
      }

      // O^T[d][qrow] = V^T[d][key] * P^T[key][qrow].  Step u covers keys of tile u/2;
      // k-slot (h, e) is key 32*(u/2) + 16*(u%2) + 4h + (e%4) + 8*(e/4).
      f32x16_t oacc[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16_t{};
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        asm volatile("" ::: "memory");  // issue this step's V^T reads just in time
        const int kt = u >> 1, hf = u & 1;
        const int key0 = kt * 32 + 16 * hf + 4 * h;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const uint8_t* vrow = Vt + (dt * 32 + l32) * kVtStride;
          const uint2 v0 = *reinterpret_cast<const uint2*>(vrow + key0 * 2);
          const uint2 v1 = *reinterpret_cast<const uint2*>(vrow + (key0 + 8) * 2);
          oacc[dt] = mfma_32x32x16(as_bf16x8(make_uint4(v0.x, v0.y, v1.x, v1.y)), as_bf16x8(pb[u]), oacc[dt]);
        }
      }

      if (valid) {
        const float inv_l = l > 0.f ? 1.f / l : 0.f;
        const int64_t prow = ((i_local * H_kv + r) * kk + s) * G + g;
        uint16_t* op = Opart + prow * kDh;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const int d0 = dt * 32 + 8 * c + 4 * h;
            uint2 pk;
            pk.x = pack_bf16x2(oacc[dt][4 * c + 0] * inv_l, oacc[dt][4 * c + 1] * inv_l);
            pk.y = pack_bf16x2(oacc[dt][4 * c + 2] * inv_l, oacc[dt][4 * c + 3] * inv_l);
            *reinterpret_cast<uint2*>(op + d0) = pk;
          }
        }
        if (h == 0) Lpart[prow] = l > 0.f ? (mx + __log2f(l)) * kLn2 : -__builtin_inff();
      }
    }
  }
}

// --------------------------------------------------------------------- phase 2
// One wave per (query, head): LSE merge of the valid slots' normalised partials.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ Opart,
                                                      const float* __restrict__ Lpart,
                                                      const int32_t* __restrict__ block_idx, int64_t w0,
                                                      int64_t W, int H_kv, int G, int kk, int64_t B,
                                                      float* __restrict__ o, float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int H_q = H_kv * G;
  if (gw >= W * H_q) return;
  const int64_t i_local = gw / H_q;
  const int hh = (int)(gw % H_q);
  const int r = hh / G, g = hh % G;
  const int64_t i = w0 + i_local;
  const int32_t* sel = block_idx + (i * H_kv + r) * kk;
  const int64_t pbase = (i_local * H_kv + r) * kk;

  float mstar = -__builtin_inff();
  for (int s = 0; s < kk; ++s) {
    if (pair_valid(sel[s], i, B)) mstar = fmaxf(mstar, Lpart[(pbase + s) * G + g]);
  }
  float* orow = o + (i * H_q + hh) * kDh;
  if (mstar == -__builtin_inff()) {
    *reinterpret_cast<float2*>(orow + 2 * lane) = make_float2(0.f, 0.f);
    if (lane == 0) lse[i * H_q + hh] = -__builtin_inff();
    return;
  }
  float a0 = 0.f, a1 = 0.f, L = 0.f;
  for (int s = 0; s < kk; ++s) {
    if (!pair_valid(sel[s], i, B)) continue;
    const int64_t prow = (pbase + s) * G + g;
    const float ls = Lpart[prow];
    if (ls == -__builtin_inff()) continue;
    const float wgt = __expf(ls - mstar);
    const uint32_t pv = *reinterpret_cast<const uint32_t*>(Opart + prow * kDh + 2 * lane);
    a0 += wgt * __uint_as_float(pv << 16);
    a1 += wgt * __uint_as_float(pv & 0xffff0000u);
    L += wgt;
  }
  const float invL = 1.f / L;
  *reinterpret_cast<float2*>(orow + 2 * lane) = make_float2(a0 * invL, a1 * invL);
  if (lane == 0) lse[i * H_q + hh] = mstar + __logf(L);
}

__global__ void fill_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t val) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += stride) p[e] = val;
}

}  // namespace

AttnWorkspace attn_workspace_layout(int64_t W, int H_q, int H_kv, int kk, int64_t B) {
  AttnWorkspace L{};
  const int64_t lists = (int64_t)H_kv * B;
  const int64_t max_pairs = W * H_kv * kk;
  const int G = H_q / H_kv;
  const int item_q = kItemChunks * (128 / G);
  const int64_t max_items = (max_pairs + item_q - 1) / item_q + lists;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~size_t(255);
    return o;
  };
  L.counts = take(sizeof(int32_t) * lists);
  L.cursor = take(sizeof(int32_t) * lists);
  L.n_items = take(sizeof(int32_t) * 4);
  L.items = take(sizeof(int4) * max_items);
  L.pairs = take(sizeof(int32_t) * max_pairs);
  L.opart = take(sizeof(uint16_t) * max_pairs * G * kDh);
  L.lpart = take(sizeof(float) * max_pairs * G);
  L.total = off;
  L.max_items = max_items;
  L.item_q = item_q;
  return L;
}

hipError_t launch_sparse_attn_window(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                     const int32_t* block_idx, int64_t N, int H_q, int H_kv, int kk,
                                     float scale, int64_t w0, int64_t W, int num_cus, float* o, float* lse,
                                     uint8_t* ws, const AttnWorkspace& L, hipStream_t stream) {
  const int64_t B = (N + kBk - 1) / kBk;
  const int64_t lists = (int64_t)H_kv * B;
  const int G = H_q / H_kv;
  int32_t* counts = reinterpret_cast<int32_t*>(ws + L.counts);
  int32_t* cursor = reinterpret_cast<int32_t*>(ws + L.cursor);
  int32_t* n_items = reinterpret_cast<int32_t*>(ws + L.n_items);
  int4* items = reinterpret_cast<int4*>(ws + L.items);
  int32_t* pairs = reinterpret_cast<int32_t*>(ws + L.pairs);
  uint16_t* opart = reinterpret_cast<uint16_t*>(ws + L.opart);
  float* lpart = reinterpret_cast<float*>(ws + L.lpart);

  fill_i32_kernel<<<dim3(256), dim3(256), 0, stream>>>(counts, lists, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // Query tiles of the inverse-index passes hold 4096 pairs (16 per thread).
  const int TQ = 4096 / kk > 0 ? 4096 / kk : 1;
  const dim3 igrid((unsigned)((W + TQ - 1) / TQ), (unsigned)H_kv);
  const size_t lds_count = sizeof(int32_t) * B;
  inv_count_kernel<<<igrid, dim3(256), lds_count, stream>>>(block_idx, w0, W, H_kv, kk, B, TQ, counts);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  inv_scan_kernel<<<dim3(1), dim3(1024), 0, stream>>>(counts, lists, L.item_q, cursor, items, n_items);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  inv_scatter_kernel<16><<<igrid, dim3(256), 2 * lds_count, stream>>>(block_idx, w0, W, H_kv, kk, B, TQ,
                                                                      cursor, pairs);
  if ((e = hipGetLastError()) != hipSuccess) return e;

  int64_t grid = (int64_t)num_cus * 2;
  if (grid > L.max_items) grid = L.max_items;
  grid = ((grid + 7) / 8) * 8;
  const float scale_log2 = scale * kLog2e;
  switch (G) {
#define MSA_ATTN_CASE(GG)                                                                            \
  case GG:                                                                                           \
    attn_kvouter_kernel<GG><<<dim3((unsigned)grid), dim3(kAttnThreads), 0, stream>>>(                \
        q, k, v, items, n_items, pairs, N, H_kv, B, kk, w0, scale_log2, opart, lpart);               \
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

  const int64_t waves = W * H_q;
  combine_kernel<<<dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream>>>(opart, lpart, block_idx, w0, W,
                                                                               H_kv, G, kk, B, o, lse);
  return hipGetLastError();
}

}  // namespace msa
