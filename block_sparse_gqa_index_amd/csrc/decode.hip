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
  float runmax = -__builtin_inff();
#pragma unroll 2
  for (int kt = 0; kt < 8; ++kt) {
    const int64_t key = b * kBk + kt * 16 + col;  // this lane's A row
    f32x4_t acc = {};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const uint4 a = key < L ? *reinterpret_cast<const uint4*>(k_idx + (j0 + key) * kDidx + ks * 32 + 8 * grp)
                              : make_uint4(0, 0, 0, 0);
      acc = mfma_16x16x32(as_bf16x8(a), as_bf16x8(qop[ks]), acc);
    }
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
  for (int64_t b = lane; b < bl; b += 64) list.offer(mrow[b], (int)b);
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

// Split-K attention for one (sequence, group, slot): G heads x one block of 128 keys.
template <int G>
__global__ __launch_bounds__(256) void dec_attn_kernel(const uint16_t* __restrict__ q,
                                                       const uint16_t* __restrict__ kc,
                                                       const uint16_t* __restrict__ vc,
                                                       const int64_t* __restrict__ cu,
                                                       const int32_t* __restrict__ block_idx, int H_kv, int kk,
                                                       float scale_log2, float* __restrict__ Opart,
                                                       float* __restrict__ Lpart) {
  __shared__ float qs[G][kDh];
  __shared__ float S[G][kBk];
  __shared__ float red[4][G][kDh];
  __shared__ float inv_l[G];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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
  const int64_t kb = (int64_t)b * kBk;
  const int nkeys = (L - kb < kBk) ? (int)(L - kb) : kBk;
  for (int e = tid; e < G * kDh; e += 256) {
    const int g = e / kDh, d = e % kDh;
    qs[g][d] = bf16_to_f32(q[((int64_t)s * H_q + r * G + g) * kDh + d]);
  }
  __syncthreads();
  // Scores: thread pair (2 keys' halves) -> key = tid/2, dims 64*(tid&1) .. +63.
  {
    const int key = tid >> 1, half = tid & 1;
    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.f;
    if (key < nkeys) {
      const uint16_t* kr = kc + ((j0 + kb + key) * H_kv + r) * kDh + 64 * half;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const uint4 u = *reinterpret_cast<const uint4*>(kr + 8 * c);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const float k0 = __uint_as_float(w[m] << 16), k1 = __uint_as_float(w[m] & 0xffff0000u);
          const int d = 64 * half + 8 * c + 2 * m;
#pragma unroll
          for (int g = 0; g < G; ++g) acc[g] += qs[g][d] * k0 + qs[g][d + 1] * k1;
        }
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float tot = acc[g] + __shfl_xor(acc[g], 1);
      if (half == 0) S[g][key] = key < nkeys ? tot * scale_log2 : -__builtin_inff();
    }
  }
  __syncthreads();
  // Softmax per head: wave w handles heads w, w+4, ...
  for (int g = wave; g < G; g += 4) {
    const float x0 = S[g][lane], x1 = S[g][lane + 64];
    const float mx = wave_max(fmaxf(x0, x1));
    const float p0 = exp2f(x0 - mx), p1 = exp2f(x1 - mx);
    const float l = wave_sum(p0 + p1);
    S[g][lane] = p0;
    S[g][lane + 64] = p1;
    if (lane == 0) {
      inv_l[g] = 1.f / l;
      lp[g] = (mx + __log2f(l)) * kLn2;
    }
  }
  __syncthreads();
  // P V: thread -> dims 2*(tid%64) .. +1, keys 32*(tid/64) .. +31.
  {
    const int dp = tid & 63, kq = tid >> 6;
    float a0[G], a1[G];
#pragma unroll
    for (int g = 0; g < G; ++g) a0[g] = a1[g] = 0.f;
    for (int kk2 = 0; kk2 < 32; ++kk2) {
      const int key = kq * 32 + kk2;
      if (key >= nkeys) break;
      const uint32_t w = *reinterpret_cast<const uint32_t*>(vc + ((j0 + kb + key) * H_kv + r) * kDh + 2 * dp);
      const float v0 = __uint_as_float(w << 16), v1 = __uint_as_float(w & 0xffff0000u);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float p = S[g][key];
        a0[g] += p * v0;
        a1[g] += p * v1;
      }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
      red[kq][g][2 * dp] = a0[g];
      red[kq][g][2 * dp + 1] = a1[g];
    }
  }
  __syncthreads();
  float* op = Opart + task * G * kDh;
  for (int e = tid; e < G * kDh; e += 256) {
    const int g = e / kDh, d = e % kDh;
    op[e] = (red[0][g][d] + red[1][g][d] + red[2][g][d] + red[3][g][d]) * inv_l[g];
  }
}

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
  const int32_t* sel = block_idx + sr * kk;
  float mstar = -__builtin_inff();
  for (int t = 0; t < kk; ++t) {
    const int b = sel[t];
    if (b >= 0 && b <= bl) mstar = fmaxf(mstar, Lpart[(sr * kk + t) * G + g]);
  }
  float* orow = o + gw * kDh;
  if (mstar == -__builtin_inff()) {
    *reinterpret_cast<float2*>(orow + 2 * lane) = make_float2(0.f, 0.f);
    if (lane == 0) lse[gw] = -__builtin_inff();
    return;
  }
  float a0 = 0.f, a1 = 0.f, Ls = 0.f;
  for (int t = 0; t < kk; ++t) {
    const int b = sel[t];
    if (!(b >= 0 && b <= bl)) continue;
    const int64_t prow = (sr * kk + t) * G + g;
    const float ls = Lpart[prow];
    if (ls == -__builtin_inff()) continue;
    const float wgt = __expf(ls - mstar);
    const float2 pv = *reinterpret_cast<const float2*>(Opart + prow * kDh + 2 * lane);
    a0 += wgt * pv.x;
    a1 += wgt * pv.y;
    Ls += wgt;
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
