// Measured-peak kernels for the benchmark (not part of the MSA library): a
// register-only bf16 MFMA loop and a streaming HBM read.  Built into its own
// libmsa_peaks.so, which only bench.py loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Each wave runs `iters` rounds of four independent 32x32x16 bf16 MFMA chains
// (32768 FLOP per MFMA); the sums are written only when `sink` asks, so the chains
// cannot be removed.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, int sink, float* out) {
  const int lane = threadIdx.x & 63;
  u32x4_t ua = {0x3f803f80u ^ (uint32_t)lane, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
  u32x4_t ub = {0x3c003c00u, 0x3c003c00u ^ (uint32_t)lane, 0x3c003c00u, 0x3c003c00u};
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, ua);
  const bf16x8_t b = __builtin_bit_cast(bf16x8_t, ub);
  f32x16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  if (sink) {
    float s = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) s += c0[v] + c1[v] + c2[v] + c3[v];
    out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  }
}

// Streaming read of n16 16-byte words (non-temporal loads, four in flight per
// thread); the XOR of everything is written only when it equals `sink`.
__global__ __launch_bounds__(256) void read_kernel(const u32x4_t* __restrict__ p, int64_t n16, uint32_t sink,
                                                   uint32_t* out) {
  int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t st = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  for (; i + 3 * st < n16; i += 4 * st) {
    const u32x4_t a = __builtin_nontemporal_load(p + i);
    const u32x4_t b = __builtin_nontemporal_load(p + i + st);
    const u32x4_t c = __builtin_nontemporal_load(p + i + 2 * st);
    const u32x4_t d = __builtin_nontemporal_load(p + i + 3 * st);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += st) {
    const u32x4_t a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == sink) out[0] = acc;
}

}  // namespace

extern "C" {

// waves_per_cu x num_cus waves of `iters` rounds; out holds one float per thread.
int msa_peak_mfma(int num_cus, int waves_per_cu, int iters, float* out, void* stream) {
  const int grid = num_cus * waves_per_cu / 4;
  mfma_loop_kernel<<<dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(iters, 0, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// Reads `bytes` (a multiple of 16) from p; out holds one uint32.
int msa_peak_read(const void* p, int64_t bytes, int num_cus, uint32_t* out, void* stream) {
  read_kernel<<<dim3(num_cus * 8), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const u32x4_t*>(p), bytes / 16, 0x9e3779b9u, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

}  // extern "C"
