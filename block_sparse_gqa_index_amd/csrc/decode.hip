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
//   3. split-K attention: one workgroup per (sequence, group, chosen block)
//      streams that block's K/V (64 KB) once for the G heads of the group.
//   4. combine: LSE merge of the k partials per (sequence, head).
#include "msa_device.h"
#include "msa_kernels.h"

namespace msa {

namespace {

constexpr int kScoreBlocksPerWG = 4;  // one block (128 keys) per wave

__global__ __launch_bounds__(256) void dec_score_kernel(const uint16_t* __restrict__ q_idx,
                                                        const uint16_t* __restrict__ k_idx,
                                                        const int64_t* __restrict__ cu, int H_kv, int64_t Bmax,
                                                        float* __restrict__ M) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int s = blockIdx.x;
  const int64_t j0 = cu[s];
  const int64_t L = cu[s + 1] - j0;
  const int64_t nb = (L + kBk - 1) / kBk;
  const int64_t b = (int64_t)blockIdx.y * kScoreBlocksPerWG + wave;
  if (b >= nb || b >= Bmax) return;
  const int col = lane & 15, grp = lane >> 4;
  uint4 qop[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
    qop[ks] = col < H_kv ? *reinterpret_cast<const uint4*>(q_idx + ((int64_t)s * H_kv + col) * kDidx + ks * 32 + 8 * grp)
                         : make_uint4(0, 0, 0, 0);
  // The block's 128 index keys (16 KB, read once per step: non-temporal) are all
  // requested before the first MFMA.  Keys past the sequence end re-read its last
  // key (a valid address); their scores are masked below.
  u32x4_t ka[8][2];
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    const int64_t key = b * kBk + kt * 16 + col;  // this lane's A row
    const int64_t kr = key < L ? key : L - 1;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
      ka[kt][ks] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4_t*>(k_idx + (j0 + kr) * kDidx + ks * 32 + 8 * grp));
  }
  float runmax = -__builtin_inff();
#pragma unroll
  for (int kt = 0; kt < 8; ++kt) {
    f32x4_t acc = {};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) acc = mfma_16x16x32(as_bf16x8(ka[kt][ks]), as_bf16x8(qop[ks]), acc);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t pos = b * kBk + kt * 16 + 4 * grp + v;
      runmax = fmaxf(runmax, pos < L ? acc[v] : -__builtin_inff());
    }
  }
  runmax = fmaxf(runmax, __shfl_xor(runmax, 16));
  runmax = fmaxf(runmax, __shfl_xor(runmax, 32));
  if (lane < 16 && col < H_kv) M[((int64_t)s * H_kv + col) * Bmax + b] = runmax * 0.125f;
}

template <int LIST>
__global__ __launch_bounds__(256) void dec_topk_kernel(const float* __restrict__ M, const int64_t* __restrict__ cu,
                                                       int batch, int H_kv, int64_t Bmax, int k,
                                                       int32_t* __restrict__ block_idx) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)batch * H_kv) return;
  const int s = (int)(row / H_kv);
  const int64_t L = cu[s + 1] - cu[s];
  int32_t* out = block_idx + row * k;
  if (L <= 0) {
    for (int t = lane; t < k; t += 64) out[t] = -1;
    return;
  }
  int64_t bl = (L - 1) / kBk;
  if (bl > Bmax - 1) bl = Bmax - 1;
  TopList<LIST> list;
  list.init();
  const float* mrow = M + row * Bmax;
  // Batches of 16 scores per lane are loaded before any is offered (the loads
  // would otherwise wait one at a time behind the list updates).
  for (int64_t b0 = 0; b0 < bl; b0 += 16 * 64) {
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t b = b0 + lane + 64 * j;
      v[j] = mrow[b < bl ? b : 0];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int64_t b = b0 + lane + 64 * j;
      if (b < bl) list.offer(v[j], (int)b);
    }
  }
  // k-1 rounds of wave arg-max over the list heads (ties: lower block index).
  int cand[LIST + 1];
#pragma unroll
  for (int t = 0; t <= LIST; ++t) cand[t] = 0x7fffffff;
#pragma unroll
  for (int t = 0; t < LIST; ++t) {
    if (t < k - 1) {
      float bv = list.v[0];
      int bb = list.b[0];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        const float ov = __shfl_xor(bv, m);
        const int ob = __shfl_xor(bb, m);
        const bool take = (ob >= 0) && (bb < 0 || ov > bv || (ov == bv && ob < bb));
        bv = take ? ov : bv;
        bb = take ? ob : bb;
      }
      if (bb >= 0) {
        cand[t] = bb;
        if (list.b[0] == bb) list.pop();
      }
    }
  }
  if (lane == 0) {
    int32_t o[LIST + 1];
    write_selection<LIST + 1>(cand, k, (int)bl, o);
#pragma unroll
    for (int t = 0; t <= LIST; ++t)
      if (t < k) out[t] = o[t];
  }
}

// Split-K attention for one (sequence, group, slot): the G heads of the group
// against one block of up to 128 keys, on 32x32x16 bf16 MFMAs.  Wave w takes keys
// 32w .. 32w+31: it reads its K rows straight into MFMA operands (S^T = K Q^T,
// heads as the 32 MFMA columns, G of them real), takes the softmax with its own
// max, and computes O^T = V^T P^T from the block's V^T, which the workgroup stages
// in LDS with coalesced 16-byte loads (non-temporal: V is read once per step).
// The four waves' (max, sum, O) are merged in LDS (rescaled to
// the common max) and the normalised partial plus its natural-log LSE is written.
// 33 KB of LDS per workgroup: four workgroups per CU keep the loads in flight.
template <int G>
__global__ __launch_bounds__(256, 4) void dec_attn_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ kc,
                                                          const uint16_t* __restrict__ vc,
                                                          const int64_t* __restrict__ cu,
                                                          const int32_t* __restrict__ block_idx, int H_kv,
                                                          int kk, float scale_log2, float* __restrict__ Opart,
                                                          float* __restrict__ Lpart) {
  static_assert(G <= 16, "the merge reuses the 32 KB V^T buffer: 4 x G x 128 fp32");
  __shared__ __attribute__((aligned(16))) uint8_t Vt[kDh * 256];  // reused for the merge
  __shared__ float wm[4][32], wl[4][32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int64_t task = blockIdx.x;  // (s * H_kv + r) * kk + slot
  const int64_t sr = task / kk;
  const int s = (int)(sr / H_kv), r = (int)(sr % H_kv);
  const int64_t j0 = cu[s];
  const int64_t L = cu[s + 1] - j0;
  const int b = block_idx[task];
  const int H_q = H_kv * G;
  float* lp = Lpart + task * G;
  if (L <= 0 || b < 0 || (int64_t)b > (L - 1) / kBk) {
    if (tid < G) lp[tid] = -__builtin_inff();
    return;
  }
  const int64_t kb0 = (int64_t)b * kBk;
  const int nvalid = (L - kb0 < kBk) ? (int)(L - kb0) : kBk;
  const int row_stride = H_kv * kDh;
  const uint16_t* kblk = kc + ((j0 + kb0) * H_kv + r) * kDh;
  // K operand of this lane: row l32 of the wave's tile is key 32w + swap23(l32)
  // (the prefill LDS order), chunk 8h + t at step t; keys past the end are clamped
  // here and masked after the scores.
  u32x4_t ka[8];
  {
    const int key = 32 * wave + swap23(l32);
    const uint16_t* kr = kblk + (key < nvalid ? key : nvalid - 1) * row_stride + 64 * h;
#pragma unroll
    for (int t = 0; t < 8; ++t) ka[t] = ld16<false>(kr + 8 * t);
  }
  stage_v<true>(vc + ((j0 + kb0) * H_kv + r) * kDh, row_stride, nvalid, Vt, tid);
  // q operand: k-slot (h, e) of step t is dim 64h + 8t + e of head l32 (zero for
  // the padding columns l32 >= G).
  u32x4_t qop[8];
  {
    const uint16_t* qr = q + ((int64_t)s * H_q + r * G + (l32 < G ? l32 : 0)) * kDh + 64 * h;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(qr + 8 * t);
      qop[t] = l32 < G ? v : u32x4_t{0u, 0u, 0u, 0u};
    }
  }

  // S^T tile of this wave: element v is key 32*wave + 16(v/8) + 4((v/4)%2) + v%4 + 8h.
  f32x16_t sacc = f32x16_t{};
#pragma unroll
  for (int t = 0; t < 8; ++t) sacc = mfma_32x32x16(as_bf16x8(ka[t]), as_bf16x8(qop[t]), sacc);
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
  const bool empty = mx == -__builtin_inff();  // every key of this wave's tile is past the end
  const float m2 = empty ? 0.f : mx * scale_log2;
  float l = 0.f;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const float p = __builtin_amdgcn_exp2f(fmaf(sacc[v], scale_log2, -m2));
    sacc[v] = p;
    l += p;
  }
  l += __shfl_xor(l, 32);
  u32x4_t pb[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    pb[hf].x = pack_bf16x2(sacc[8 * hf + 0], sacc[8 * hf + 1]);
    pb[hf].y = pack_bf16x2(sacc[8 * hf + 2], sacc[8 * hf + 3]);
    pb[hf].z = pack_bf16x2(sacc[8 * hf + 4], sacc[8 * hf + 5]);
    pb[hf].w = pack_bf16x2(sacc[8 * hf + 6], sacc[8 * hf + 7]);
  }
  __syncthreads();  // V^T staged
  // O^T[d][head] over this wave's keys: steps u = 2*wave + hf, V^T chunk 2u + h.
  f32x16_t oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16_t{};
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int kc2 = 2 * (2 * wave + hf) + h;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int d = dt * 32 + l32;
      const u32x4_t va = *reinterpret_cast<const u32x4_t*>(Vt + d * 256 + ((kc2 ^ (d & 15)) << 4));
      oacc[dt] = mfma_32x32x16(as_bf16x8(va), as_bf16x8(pb[hf]), oacc[dt]);
    }
  }
  if (h == 0) {
    wm[wave][l32] = empty ? -__builtin_inff() : m2;
    wl[wave][l32] = l;
  }
  __syncthreads();  // every wave is done with V^T
  // Merge: the four waves' O^T for the G real heads, rescaled to the common max.
  float* red = reinterpret_cast<float*>(Vt);  // [4][G][128]
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
    op[e] = acc / ls;
    if (d == 0) lp[g] = (M + __log2f(ls)) * kLn2;
  }
}

// LSE merge of the k slot partials of one (sequence, head) per wave.  Lane t < k
// reads slot t's block index and LSE (validity, the common max and each slot's
// weight are then wave reductions and lane reads); lane j then accumulates dims
// 2j, 2j+1 over the slots, with every slot's row load independent of the others.
__global__ __launch_bounds__(256) void dec_combine_kernel(const float* __restrict__ Opart,
                                                          const float* __restrict__ Lpart,
                                                          const int32_t* __restrict__ block_idx,
                                                          const int64_t* __restrict__ cu, int batch, int H_kv,
                                                          int G, int kk, float* __restrict__ o,
                                                          float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t gw = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int H_q = H_kv * G;
  if (gw >= (int64_t)batch * H_q) return;
  const int s = (int)(gw / H_q), hh = (int)(gw % H_q);
  const int r = hh / G, g = hh % G;
  const int64_t L = cu[s + 1] - cu[s];
  const int64_t bl = L > 0 ? (L - 1) / kBk : -1;
  const int64_t sr = (int64_t)s * H_kv + r;
  const int t = lane < kk ? lane : 0;
  const int b = block_idx[sr * kk + t];
  const float ls = Lpart[(sr * kk + t) * G + g];
  const bool valid = lane < kk && b >= 0 && b <= bl && ls != -__builtin_inff();
  const float mstar = wave_max(valid ? ls : -__builtin_inff());
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
  for (int u = 0; u < kk; ++u) {
    const float wu = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wgt), u));
    // Rows of invalid slots were never written: read the first valid slot's row
    // instead (weight 0).
    const int us = ((vm >> u) & 1) ? u : first;
    const float2 pv = *reinterpret_cast<const float2*>(Opart + ((sr * kk + us) * G + g) * kDh + 2 * lane);
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
  L.opart = take(sizeof(float) * (size_t)batch * H_kv * kk * G * kDh);
  L.lpart = take(sizeof(float) * (size_t)batch * H_kv * kk * G);
  L.total = off;
  return L;
}

hipError_t launch_decode(const uint16_t* q, const uint16_t* q_idx, const uint16_t* k_cache,
                         const uint16_t* v_cache, const uint16_t* k_idx_cache, const int64_t* cu, int batch,
                         int64_t Bmax, int H_q, int H_kv, int kk, float scale, int32_t* block_idx, float* o,
                         float* lse, uint8_t* ws, const DecodeWorkspace& L, hipStream_t stream) {
  const int G = H_q / H_kv;
  float* M = reinterpret_cast<float*>(ws + L.M);
  float* opart = reinterpret_cast<float*>(ws + L.opart);
  float* lpart = reinterpret_cast<float*>(ws + L.lpart);
  hipError_t e;
  dec_score_kernel<<<dim3((unsigned)batch, (unsigned)((Bmax + kScoreBlocksPerWG - 1) / kScoreBlocksPerWG)),
                     dim3(256), 0, stream>>>(q_idx, k_idx_cache, cu, H_kv, Bmax, M);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const unsigned rows_grid = (unsigned)(((int64_t)batch * H_kv + 3) / 4);
  if (kk <= 8)
    dec_topk_kernel<7><<<dim3(rows_grid), dim3(256), 0, stream>>>(M, cu, batch, H_kv, Bmax, kk, block_idx);
  else if (kk <= 16)
    dec_topk_kernel<15><<<dim3(rows_grid), dim3(256), 0, stream>>>(M, cu, batch, H_kv, Bmax, kk, block_idx);
  else
    dec_topk_kernel<31><<<dim3(rows_grid), dim3(256), 0, stream>>>(M, cu, batch, H_kv, Bmax, kk, block_idx);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const float scale_log2 = scale * kLog2e;
  const unsigned tasks = (unsigned)((int64_t)batch * H_kv * kk);
  switch (G) {
#define MSA_DEC_CASE(GG)                                                                              \
  case GG:                                                                                            \
    dec_attn_kernel<GG><<<dim3(tasks), dim3(256), 0, stream>>>(q, k_cache, v_cache, cu, block_idx, H_kv, \
                                                               kk, scale_log2, opart, lpart);          \
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
  dec_combine_kernel<<<dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream>>>(opart, lpart, block_idx, cu,
                                                                                  batch, H_kv, G, kk, o, lse);
  return hipGetLastError();
}

}  // namespace msa
