// C ABI of the MSA forward path: argument checks, workspace sizing and launches.
// Every entry point validates on the host, then enqueues asynchronously on the
// caller's stream; nothing here synchronises or allocates device memory.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "msa.h"
#include "msa_kernels.h"

// Device memory of msa_decode_noalloc: one copy per GPU, created when the library's
// code object is loaded on that GPU and held until the process ends.  In host code
// `scratch` only names the symbol; its device address on the current GPU comes from
// hipGetSymbolAddress (scratch_on_current_device below).
static __device__ __align__(256) uint8_t scratch[MSA_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[512] = "";
// Caller-owned events recorded at the phase boundaries of msa_sparse_attn_fwd.
constexpr int kMaxProfileWindows = 1024;
thread_local hipEvent_t g_phase_events[4 * kMaxProfileWindows] = {};
thread_local int g_phase_windows = 0;  // windows with events; 0 = hook off
// Per-workgroup clock buffer of the persistent-grid kernels (msa_set_profile_clock).
thread_local uint64_t* g_clock = nullptr;
thread_local int64_t g_clock_slots = 0;

msa_status_t fail(msa_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

msa_status_t ok() {
  g_last_error[0] = '\0';
  return MSA_OK;
}

msa_status_t hip_fail(hipError_t e, const char* where) {
  return fail(MSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

constexpr int64_t kMaxN = (int64_t)1 << 24;
constexpr int64_t kMaxBlocks = 8192;  // inverse-index passes keep 2 x B counters in LDS
// Default cap on the KV-outer partial buffers; larger inputs run in query windows.
constexpr size_t kDefaultAttnWorkspace = (size_t)40 << 30;
// The backward's default is larger: at 128K (H_q = 64, H_kv = 8, k = 16) it then runs
// in one query window (measured 52.2 ms against 54.4 ms for two under 40 GiB).
constexpr size_t kDefaultBwdWorkspace = (size_t)64 << 30;

msa_status_t check_common(int64_t N, int d, int expect_d, const char* dname, int B_k, int k) {
  if (N < 0) return fail(MSA_ERR_INVALID_ARG, "N must be >= 0 (got %lld)", (long long)N);
  if (d != expect_d) return fail(MSA_ERR_UNSUPPORTED, "%s must be %d (got %d)", dname, expect_d, d);
  if (B_k != 64 && B_k != 128) return fail(MSA_ERR_UNSUPPORTED, "B_k must be 64 or 128 (got %d)", B_k);
  if (k < 1 || k > 32) return fail(MSA_ERR_UNSUPPORTED, "k must be in [1, 32] (got %d)", k);
  if (N >= kMaxN) return fail(MSA_ERR_UNSUPPORTED, "N must be < 2^24 (got %lld)", (long long)N);
  if ((N + B_k - 1) / B_k > kMaxBlocks) return fail(MSA_ERR_UNSUPPORTED, "too many blocks");
  return MSA_OK;
}

// Device address of `scratch` per device ordinal, looked up on the first
// msa_decode_noalloc call made with that device current.
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxScratchDevices] = {};

msa_status_t scratch_on_current_device(uint8_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MSA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(MSA_ERR_UNSUPPORTED, "device ordinal %d is above %d", dev, kMaxScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(MSA_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}

int num_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Largest query window (whole blocks of queries, at least one block) whose
// per-window workspace fits in ws_bytes; B is the list stride in blocks.
int64_t window_for_bytes(int64_t N, int64_t B, int H_q, int H_kv, int k, size_t ws_bytes, int parts = msa::kPartsAttn) {
  int64_t lo = 0, hi = (N + msa::kBlockKeys - 1) / msa::kBlockKeys;
  while (lo < hi) {
    const int64_t mid = (lo + hi + 1) / 2;
    const int64_t W = mid * msa::kBlockKeys < N ? mid * msa::kBlockKeys : N;
    if (msa::attn_workspace_layout(W, H_q, H_kv, k, B, parts).total <= ws_bytes)
      lo = mid;
    else
      hi = mid - 1;
  }
  const int64_t W = lo * msa::kBlockKeys < N ? lo * msa::kBlockKeys : N;
  const int64_t Wmin = N < msa::kBlockKeys ? N : msa::kBlockKeys;
  return W > Wmin ? W : Wmin;
}

}  // namespace

extern "C" {

const char* msa_status_string(msa_status_t s) {
  switch (s) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARG: return "MSA_ERR_INVALID_ARG";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED";
    case MSA_ERR_WORKSPACE: return "MSA_ERR_WORKSPACE";
    case MSA_ERR_HIP: return "MSA_ERR_HIP";
  }
  return "MSA_ERR_UNKNOWN";
}

const char* msa_last_error(void) { return g_last_error; }

size_t msa_index_topk_workspace(int64_t, int, int, int, int) { return 0; }

msa_status_t msa_index_topk(const void* q_idx, const void* k_idx, int64_t N, int H_kv, int d_idx, int B_k, int k,
                            int32_t* block_idx, void*, size_t, void* hip_stream) {
  msa_status_t st = check_common(N, d_idx, msa::kIndexDim, "d_idx", B_k, k);
  if (st != MSA_OK) return st;
  if (H_kv < 1) return fail(MSA_ERR_INVALID_ARG, "H_kv must be >= 1");
  if (N == 0) return ok();
  if (!q_idx || !k_idx || !block_idx) return fail(MSA_ERR_INVALID_ARG, "null pointer");
  if (!aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(block_idx, 4))
    return fail(MSA_ERR_INVALID_ARG, "misaligned pointer (q_idx/k_idx need 16 B, block_idx 4 B)");
  if (N * H_kv >= ((int64_t)1 << 31)) return fail(MSA_ERR_UNSUPPORTED, "N * H_kv too large");
  hipError_t e = msa::launch_index_topk(static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_idx),
                                        N, H_kv, k, block_idx, nullptr, 0, N, B_k, num_cus(),
                                        static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "index_topk launch");
  return ok();
}

msa_status_t msa_index_block_scores(const void* q_idx, const void* k_idx, int64_t N, int H_kv, int d_idx, int B_k,
                                    float* M, void* hip_stream) {
  msa_status_t st = check_common(N, d_idx, msa::kIndexDim, "d_idx", B_k, 1);
  if (st != MSA_OK) return st;
  if (H_kv < 1) return fail(MSA_ERR_INVALID_ARG, "H_kv must be >= 1");
  if (N == 0) return ok();
  if (!q_idx || !k_idx || !M) return fail(MSA_ERR_INVALID_ARG, "null pointer");
  if (!aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(M, 4))
    return fail(MSA_ERR_INVALID_ARG, "misaligned pointer");
  hipError_t e = msa::launch_index_block_scores(static_cast<const uint16_t*>(q_idx),
                                                static_cast<const uint16_t*>(k_idx), N, H_kv, B_k, M,
                                                static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "index_block_scores launch");
  return ok();
}

msa_status_t msa_topk_from_scores(const float* M, int64_t N, int H_kv, int64_t B, int B_k, int k, int32_t* block_idx,
                                  void* hip_stream) {
  msa_status_t st = check_common(N, msa::kIndexDim, msa::kIndexDim, "d_idx", B_k, k);
  if (st != MSA_OK) return st;
  if (H_kv < 1) return fail(MSA_ERR_INVALID_ARG, "H_kv must be >= 1");
  if (B < (N + B_k - 1) / B_k) return fail(MSA_ERR_INVALID_ARG, "B must be >= ceil(N / B_k)");
  if (N == 0) return ok();
  if (!M || !block_idx) return fail(MSA_ERR_INVALID_ARG, "null pointer");
  if (!aligned(M, 4) || !aligned(block_idx, 4)) return fail(MSA_ERR_INVALID_ARG, "misaligned pointer");
  hipError_t e =
      msa::launch_topk_from_scores(M, N, H_kv, B, k, B_k, block_idx, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "topk_from_scores launch");
  return ok();
}

static msa_status_t check_attn_shape(int64_t N, int H_q, int H_kv, int d_h, int B_k, int k) {
  msa_status_t st = check_common(N, d_h, msa::kHeadDim, "d_h", B_k, k);
  if (st != MSA_OK) return st;
  if (H_kv < 1 || H_q < 1 || H_q % H_kv != 0)
    return fail(MSA_ERR_INVALID_ARG, "H_q must be a positive multiple of H_kv");
  const int G = H_q / H_kv;
  if (!is_pow2(G) || G > 128) return fail(MSA_ERR_UNSUPPORTED, "H_q / H_kv must be a power of two <= 128");
  if (N * H_kv >= ((int64_t)1 << 31)) return fail(MSA_ERR_UNSUPPORTED, "N * H_kv too large");
  return MSA_OK;
}

// The clock buffer when it holds 2 slots for each of up to max_wg workgroups.
static uint64_t* clock_for(int64_t max_wg) { return g_clock && g_clock_slots >= 2 * max_wg ? g_clock : nullptr; }

// Attention over N tokens with list stride B (blocks), given sequence tables si (si.cu
// null: one sequence).  The workspace holds the sequence tables (S) and then the
// per-window buffers.
static msa_status_t attn_run(const void* q, const void* k, const void* v, const int32_t* block_idx, int64_t N,
                             int64_t B, const msa::SeqInfo& si, const msa::SeqTables& S, int B_k, int H_q, int H_kv,
                             int k_sel, float scale, float* o, float* lse, uint8_t* ws, size_t ws_bytes,
                             hipStream_t stream, const void* q_idx = nullptr, const void* k_idx = nullptr,
                             float* lse_idx = nullptr) {
  const size_t avail = ws_bytes - S.total;
  const int64_t W = window_for_bytes(N, B, H_q, H_kv, k_sel, avail);
  const msa::AttnWorkspace L = msa::attn_workspace_layout(W, H_q, H_kv, k_sel, B);
  const int cus = num_cus();
  int64_t wi = 0;
  for (int64_t w0 = 0; w0 < N; w0 += W, ++wi) {
    const int64_t Wn = (N - w0 < W) ? N - w0 : W;
    hipError_t e = msa::launch_sparse_attn_window(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), block_idx,
        N, B, si, B_k, H_q, H_kv, k_sel, scale, w0, Wn, cus, o, lse, ws + S.total, L, stream,
        wi < g_phase_windows ? g_phase_events + 4 * wi : nullptr, wi == 0 ? clock_for(2 * cus + 8) : nullptr,
        static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_idx), lse_idx);
    if (e != hipSuccess) return hip_fail(e, "sparse_attn launch");
  }
  return ok();
}

static size_t attn_workspace_bytes(int64_t N, int64_t B, const msa::SeqTables& S, int H_q, int H_kv, int k,
                                   bool minimum) {
  const int64_t Wmin = N < msa::kBlockKeys ? N : msa::kBlockKeys;
  const int64_t W = minimum ? Wmin : window_for_bytes(N, B, H_q, H_kv, k, kDefaultAttnWorkspace);
  return S.total + msa::attn_workspace_layout(W, H_q, H_kv, k, B).total;
}

static msa_status_t check_attn_ptrs(const void* q, const void* k, const void* v, const int32_t* block_idx,
                                    const float* o, const float* lse, float scale) {
  if (!(scale > 0.f) || scale != scale) return fail(MSA_ERR_INVALID_ARG, "scale must be a positive number");
  if (!q || !k || !v || !block_idx || !o || !lse) return fail(MSA_ERR_INVALID_ARG, "null pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(block_idx, 4) || !aligned(o, 16) ||
      !aligned(lse, 4))
    return fail(MSA_ERR_INVALID_ARG, "misaligned pointer (q/k/v/o need 16 B)");
  return MSA_OK;
}

size_t msa_sparse_attn_fwd_workspace(int64_t N, int H_q, int H_kv, int d_h, int B_k, int k) {
  if (check_attn_shape(N, H_q, H_kv, d_h, B_k, k) != MSA_OK || N == 0) return 0;
  return attn_workspace_bytes(N, (N + B_k - 1) / B_k, msa::SeqTables{}, H_q, H_kv, k, false);
}

size_t msa_sparse_attn_fwd_workspace_min(int64_t N, int H_q, int H_kv, int d_h, int B_k, int k) {
  if (check_attn_shape(N, H_q, H_kv, d_h, B_k, k) != MSA_OK || N == 0) return 0;
  return attn_workspace_bytes(N, (N + B_k - 1) / B_k, msa::SeqTables{}, H_q, H_kv, k, true);
}

int64_t msa_sparse_attn_fwd_windows(int64_t N, int H_q, int H_kv, int d_h, int B_k, int k, size_t ws_bytes) {
  if (check_attn_shape(N, H_q, H_kv, d_h, B_k, k) != MSA_OK) return -1;
  if (N == 0) return 0;
  if (ws_bytes < msa_sparse_attn_fwd_workspace_min(N, H_q, H_kv, d_h, B_k, k)) return -1;
  const int64_t W = window_for_bytes(N, (N + B_k - 1) / B_k, H_q, H_kv, k, ws_bytes);
  return (N + W - 1) / W;
}

msa_status_t msa_sparse_attn_fwd(const void* q, const void* k, const void* v, const int32_t* block_idx, int64_t N,
                                 int H_q, int H_kv, int d_h, int B_k, int k_sel, float scale, float* o, float* lse,
                                 void* ws, size_t ws_bytes, void* hip_stream) {
  msa_status_t st = check_attn_shape(N, H_q, H_kv, d_h, B_k, k_sel);
  if (st != MSA_OK) return st;
  if (!(scale > 0.f) || scale != scale) return fail(MSA_ERR_INVALID_ARG, "scale must be a positive number");
  if (N == 0) return ok();
  if ((st = check_attn_ptrs(q, k, v, block_idx, o, lse, scale)) != MSA_OK) return st;
  const size_t need = msa_sparse_attn_fwd_workspace_min(N, H_q, H_kv, d_h, B_k, k_sel);
  if (!ws || ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes is below the minimum %zu", ws ? ws_bytes : 0, need);
  if (!aligned(ws, 256)) return fail(MSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return attn_run(q, k, v, block_idx, N, (N + B_k - 1) / B_k, msa::SeqInfo{}, msa::SeqTables{}, B_k, H_q, H_kv, k_sel,
                  scale, o, lse, static_cast<uint8_t*>(ws), ws_bytes, static_cast<hipStream_t>(hip_stream));
}

msa_status_t msa_sparse_attn_fwd_lse_idx(const void* q, const void* k, const void* v, const void* q_idx,
                                         const void* k_idx, const int32_t* block_idx, int64_t N, int H_q, int H_kv,
                                         int d_h, int d_idx, int B_k, int k_sel, float scale, float* o, float* lse,
                                         float* lse_idx, void* ws, size_t ws_bytes, void* hip_stream) {
  msa_status_t st = check_attn_shape(N, H_q, H_kv, d_h, B_k, k_sel);
  if (st != MSA_OK) return st;
  if (d_idx != msa::kIndexDim) return fail(MSA_ERR_UNSUPPORTED, "d_idx must be %d (got %d)", msa::kIndexDim, d_idx);
  if (!(scale > 0.f) || scale != scale) return fail(MSA_ERR_INVALID_ARG, "scale must be a positive number");
  if (N == 0) return ok();
  if ((st = check_attn_ptrs(q, k, v, block_idx, o, lse, scale)) != MSA_OK) return st;
  if (!q_idx || !k_idx || !lse_idx) return fail(MSA_ERR_INVALID_ARG, "null pointer");
  if (!aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(lse_idx, 4))
    return fail(MSA_ERR_INVALID_ARG, "misaligned pointer (q_idx/k_idx need 16 B)");
  const size_t need = msa_sparse_attn_fwd_workspace_min(N, H_q, H_kv, d_h, B_k, k_sel);
  if (!ws || ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes is below the minimum %zu", ws ? ws_bytes : 0, need);
  if (!aligned(ws, 256)) return fail(MSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return attn_run(q, k, v, block_idx, N, (N + B_k - 1) / B_k, msa::SeqInfo{}, msa::SeqTables{}, B_k, H_q, H_kv, k_sel,
                  scale, o, lse, static_cast<uint8_t*>(ws), ws_bytes, static_cast<hipStream_t>(hip_stream), q_idx,
                  k_idx, lse_idx);
}

// ---------------------------------------------------------------- packed sequences
static msa_status_t check_varlen(int batch, int64_t T, int64_t max_len, int B_k) {
  if (batch < 0) return fail(MSA_ERR_INVALID_ARG, "batch must be >= 0");
  if (T < 0 || max_len < 0) return fail(MSA_ERR_INVALID_ARG, "T and max_len must be >= 0");
  if (max_len > T) return fail(MSA_ERR_INVALID_ARG, "max_len must be <= T");
  if ((T + B_k - 1) / B_k + batch > kMaxBlocks)
    return fail(MSA_ERR_UNSUPPORTED, "ceil(T / B_k) + batch must be <= %lld", (long long)kMaxBlocks);
  return MSA_OK;
}

static int64_t varlen_blocks(int64_t T, int batch, int B_k) { return (T + B_k - 1) / B_k + batch; }

msa_status_t msa_index_topk_varlen(const void* q_idx, const void* k_idx, const int64_t* cu_seqlens, int batch,
                                   int64_t T, int64_t max_len, int H_kv, int d_idx, int B_k, int k,
                                   int32_t* block_idx, void* hip_stream) {
  msa_status_t st = check_common(T, d_idx, msa::kIndexDim, "d_idx", B_k, k);
  if (st != MSA_OK) return st;
  if ((st = check_varlen(batch, T, max_len, B_k)) != MSA_OK) return st;
  if (batch > 0 && T > 0 && max_len == 0) return fail(MSA_ERR_INVALID_ARG, "max_len must be >= 1");
  if (H_kv < 1) return fail(MSA_ERR_INVALID_ARG, "H_kv must be >= 1");
  if (batch == 0 || T == 0) return ok();
  if (!q_idx || !k_idx || !block_idx || !cu_seqlens) return fail(MSA_ERR_INVALID_ARG, "null pointer");
  if (!aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(block_idx, 4) || !aligned(cu_seqlens, 8))
    return fail(MSA_ERR_INVALID_ARG, "misaligned pointer");
  if (T * H_kv >= ((int64_t)1 << 31)) return fail(MSA_ERR_UNSUPPORTED, "T * H_kv too large");
  if (batch > 65535) return fail(MSA_ERR_UNSUPPORTED, "batch must be <= 65535");
  hipError_t e = msa::launch_index_topk(static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_idx),
                                        max_len, H_kv, k, block_idx, cu_seqlens, batch, T, B_k, num_cus(),
                                        static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "index_topk launch");
  return ok();
}

size_t msa_sparse_attn_fwd_varlen_workspace(int64_t T, int batch, int H_q, int H_kv, int d_h, int B_k, int k) {
  if (check_attn_shape(T, H_q, H_kv, d_h, B_k, k) != MSA_OK || check_varlen(batch, T, 0, B_k) != MSA_OK || T == 0 ||
      batch == 0)
    return 0;
  const int64_t Bt = varlen_blocks(T, batch, B_k);
  return attn_workspace_bytes(T, Bt, msa::seq_tables_layout(T, batch, Bt), H_q, H_kv, k, false);
}

size_t msa_sparse_attn_fwd_varlen_workspace_min(int64_t T, int batch, int H_q, int H_kv, int d_h, int B_k, int k) {
  if (check_attn_shape(T, H_q, H_kv, d_h, B_k, k) != MSA_OK || check_varlen(batch, T, 0, B_k) != MSA_OK || T == 0 ||
      batch == 0)
    return 0;
  const int64_t Bt = varlen_blocks(T, batch, B_k);
  return attn_workspace_bytes(T, Bt, msa::seq_tables_layout(T, batch, Bt), H_q, H_kv, k, true);
}

msa_status_t msa_sparse_attn_fwd_varlen(const void* q, const void* k, const void* v, const int32_t* block_idx,
                                        const int64_t* cu_seqlens, int batch, int64_t T, int H_q, int H_kv, int d_h,
                                        int B_k, int k_sel, float scale, float* o, float* lse, void* ws,
                                        size_t ws_bytes, void* hip_stream) {
  msa_status_t st = check_attn_shape(T, H_q, H_kv, d_h, B_k, k_sel);
  if (st != MSA_OK) return st;
  if ((st = check_varlen(batch, T, 0, B_k)) != MSA_OK) return st;
  if (!(scale > 0.f) || scale != scale) return fail(MSA_ERR_INVALID_ARG, "scale must be a positive number");
  if (batch == 0 || T == 0) return ok();
  if ((st = check_attn_ptrs(q, k, v, block_idx, o, lse, scale)) != MSA_OK) return st;
  if (!cu_seqlens) return fail(MSA_ERR_INVALID_ARG, "null pointer");
  if (!aligned(cu_seqlens, 8)) return fail(MSA_ERR_INVALID_ARG, "misaligned pointer");
  const size_t need = msa_sparse_attn_fwd_varlen_workspace_min(T, batch, H_q, H_kv, d_h, B_k, k_sel);
  if (!ws || ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes is below the minimum %zu", ws ? ws_bytes : 0, need);
  if (!aligned(ws, 256)) return fail(MSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const int64_t Bt = varlen_blocks(T, batch, B_k);
  const msa::SeqTables S = msa::seq_tables_layout(T, batch, Bt);
  uint8_t* w = static_cast<uint8_t*>(ws);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  hipError_t e = msa::launch_seq_tables(cu_seqlens, batch, T, B_k, w, S, stream);
  if (e != hipSuccess) return hip_fail(e, "sequence tables launch");
  msa::SeqInfo si;
  si.cu = reinterpret_cast<const int64_t*>(w + S.cu);  // the sanitised copy
  si.bstart = reinterpret_cast<const int32_t*>(w + S.bstart);
  si.seq_tok = reinterpret_cast<const int32_t*>(w + S.seq_tok);
  si.seq_blk = reinterpret_cast<const int32_t*>(w + S.seq_blk);
  return attn_run(q, k, v, block_idx, T, Bt, si, S, B_k, H_q, H_kv, k_sel, scale, o, lse, w, ws_bytes, stream);
}

// ---------------------------------------------------------------- KL alignment
static constexpr size_t kKlLossBytes = sizeof(double) * msa::kKlLossParts;

static size_t kl_workspace_bytes(int64_t N, int H_q, int H_kv, int k, int B_k, bool minimum) {
  const int64_t B = (N + B_k - 1) / B_k;
  const int64_t Wmin = N < msa::kBlockKeys ? N : msa::kBlockKeys;
  const int64_t W = minimum ? Wmin : window_for_bytes(N, B, H_q, H_kv, k, kDefaultAttnWorkspace, msa::kPartsKl);
  return kKlLossBytes + msa::attn_workspace_layout(W, H_q, H_kv, k, B, msa::kPartsKl).total;
}

static msa_status_t check_kl_shape(int64_t N, int H_q, int H_kv, int d_h, int d_idx, int B_k, int k) {
  msa_status_t st = check_attn_shape(N, H_q, H_kv, d_h, B_k, k);
  if (st != MSA_OK) return st;
  if (d_idx != msa::kIndexDim) return fail(MSA_ERR_UNSUPPORTED, "d_idx must be %d (got %d)", msa::kIndexDim, d_idx);
  if (H_q / H_kv > 32) return fail(MSA_ERR_UNSUPPORTED, "G = H_q / H_kv must be <= 32 for the KL pass");
  return MSA_OK;
}

size_t msa_sparse_kl_fwd_workspace(int64_t N, int H_q, int H_kv, int d_h, int d_idx, int B_k, int k) {
  if (check_kl_shape(N, H_q, H_kv, d_h, d_idx, B_k, k) != MSA_OK || N == 0) return 0;
  return kl_workspace_bytes(N, H_q, H_kv, k, B_k, false);
}

size_t msa_sparse_kl_fwd_workspace_min(int64_t N, int H_q, int H_kv, int d_h, int d_idx, int B_k, int k) {
  if (check_kl_shape(N, H_q, H_kv, d_h, d_idx, B_k, k) != MSA_OK || N == 0) return 0;
  return kl_workspace_bytes(N, H_q, H_kv, k, B_k, true);
}

// msa_sparse_kl_fwd and msa_sparse_kl_fwd_from_lse_idx: lse_idx_in null computes
// LSE_idx into lse_idx; otherwise LSE_idx is read from lse_idx_in (lse_idx unused).
static msa_status_t sparse_kl_run(const void* q, const void* k, const void* q_idx, const void* k_idx,
                                  const int32_t* block_idx, const float* lse, const float* lse_idx_in, int64_t N,
                                  int H_q, int H_kv, int d_h, int d_idx, int B_k, int k_sel, float scale, float* kl,
                                  float* lse_idx, float* loss, void* ws, size_t ws_bytes, void* hip_stream) {
  msa_status_t st = check_kl_shape(N, H_q, H_kv, d_h, d_idx, B_k, k_sel);
  if (st != MSA_OK) return st;
  if (!(scale > 0.f) || scale != scale) return fail(MSA_ERR_INVALID_ARG, "scale must be a positive number");
  if (N == 0) return ok();
  if (!q || !k || !q_idx || !k_idx || !block_idx || !lse || !kl || !(lse_idx || lse_idx_in) || !loss)
    return fail(MSA_ERR_INVALID_ARG, "null pointer");
  const void* li = lse_idx_in ? static_cast<const void*>(lse_idx_in) : static_cast<const void*>(lse_idx);
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(q_idx, 16) || !aligned(k_idx, 16) || !aligned(block_idx, 4) ||
      !aligned(lse, 4) || !aligned(kl, 4) || !aligned(li, 4) || !aligned(loss, 4))
    return fail(MSA_ERR_INVALID_ARG, "misaligned pointer (q/k/q_idx/k_idx need 16 B)");
  const size_t need = msa_sparse_kl_fwd_workspace_min(N, H_q, H_kv, d_h, d_idx, B_k, k_sel);
  if (!ws || ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes is below the minimum %zu", ws ? ws_bytes : 0, need);
  if (!aligned(ws, 256)) return fail(MSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const int64_t B = (N + B_k - 1) / B_k;
  uint8_t* w = static_cast<uint8_t*>(ws);
  const int64_t W = window_for_bytes(N, B, H_q, H_kv, k_sel, ws_bytes - kKlLossBytes, msa::kPartsKl);
  const msa::AttnWorkspace L = msa::attn_workspace_layout(W, H_q, H_kv, k_sel, B, msa::kPartsKl);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  const int cus = num_cus();
  for (int64_t w0 = 0; w0 < N; w0 += W) {
    const int64_t Wn = (N - w0 < W) ? N - w0 : W;
    hipError_t e = msa::launch_sparse_kl_window(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(q_idx),
        static_cast<const uint16_t*>(k_idx), lse, block_idx, N, B, B_k, H_q, H_kv, k_sel, scale, w0, Wn, cus,
        lse_idx_in, kl, lse_idx, w + kKlLossBytes, L, stream);
    if (e != hipSuccess) return hip_fail(e, "sparse_kl launch");
  }
  hipError_t e = msa::launch_kl_loss(kl, N * H_kv, reinterpret_cast<double*>(w), loss, stream);
  if (e != hipSuccess) return hip_fail(e, "kl loss launch");
  return ok();
}

msa_status_t msa_sparse_kl_fwd(const void* q, const void* k, const void* q_idx, const void* k_idx,
                               const int32_t* block_idx, const float* lse, int64_t N, int H_q, int H_kv, int d_h,
                               int d_idx, int B_k, int k_sel, float scale, float* kl, float* lse_idx, float* loss,
                               void* ws, size_t ws_bytes, void* hip_stream) {
  return sparse_kl_run(q, k, q_idx, k_idx, block_idx, lse, nullptr, N, H_q, H_kv, d_h, d_idx, B_k, k_sel, scale, kl,
                       lse_idx, loss, ws, ws_bytes, hip_stream);
}

msa_status_t msa_sparse_kl_fwd_from_lse_idx(const void* q, const void* k, const void* q_idx, const void* k_idx,
                                            const int32_t* block_idx, const float* lse, const float* lse_idx,
                                            int64_t N, int H_q, int H_kv, int d_h, int d_idx, int B_k, int k_sel,
                                            float scale, float* kl, float* loss, void* ws, size_t ws_bytes,
                                            void* hip_stream) {
  return sparse_kl_run(q, k, q_idx, k_idx, block_idx, lse, lse_idx, N, H_q, H_kv, d_h, d_idx, B_k, k_sel, scale, kl,
                       nullptr, loss, ws, ws_bytes, hip_stream);
}

// ---------------------------------------------------------------- backward
static size_t bwd_d_bytes(int64_t N, int H_q) { return ((sizeof(float) * (size_t)N * H_q) + 255) & ~size_t(255); }

static msa_status_t check_bwd_shape(int64_t N, int H_q, int H_kv, int d_h, int B_k, int k) {
  msa_status_t st = check_attn_shape(N, H_q, H_kv, d_h, B_k, k);
  if (st != MSA_OK) return st;
  if (H_q / H_kv > 32) return fail(MSA_ERR_UNSUPPORTED, "the backward supports G = H_q / H_kv <= 32");
  return MSA_OK;
}

static size_t bwd_workspace_bytes(int64_t N, int H_q, int H_kv, int k, int B_k, bool minimum) {
  const int64_t B = (N + B_k - 1) / B_k;
  const int64_t Wmin = N < msa::kBlockKeys ? N : msa::kBlockKeys;
  const int64_t W = minimum ? Wmin : window_for_bytes(N, B, H_q, H_kv, k, kDefaultBwdWorkspace, msa::kPartsBwd);
  return bwd_d_bytes(N, H_q) + msa::attn_workspace_layout(W, H_q, H_kv, k, B, msa::kPartsBwd).total;
}

size_t msa_sparse_attn_bwd_workspace(int64_t N, int H_q, int H_kv, int d_h, int B_k, int k) {
  if (check_bwd_shape(N, H_q, H_kv, d_h, B_k, k) != MSA_OK || N == 0) return 0;
  return bwd_workspace_bytes(N, H_q, H_kv, k, B_k, false);
}

size_t msa_sparse_attn_bwd_workspace_min(int64_t N, int H_q, int H_kv, int d_h, int B_k, int k) {
  if (check_bwd_shape(N, H_q, H_kv, d_h, B_k, k) != MSA_OK || N == 0) return 0;
  return bwd_workspace_bytes(N, H_q, H_kv, k, B_k, true);
}

msa_status_t msa_sparse_attn_bwd(const void* q, const void* k, const void* v, const float* o, const float* lse,
                                 const void* dO, const int32_t* block_idx, int64_t N, int H_q, int H_kv, int d_h,
                                 int B_k, int k_sel, float scale, float* dq, float* dk, float* dv, void* ws,
                                 size_t ws_bytes, void* hip_stream) {
  msa_status_t st = check_bwd_shape(N, H_q, H_kv, d_h, B_k, k_sel);
  if (st != MSA_OK) return st;
  if (!(scale > 0.f) || scale != scale) return fail(MSA_ERR_INVALID_ARG, "scale must be a positive number");
  if (N == 0) return ok();
  if (!q || !k || !v || !o || !lse || !dO || !block_idx || !dq || !dk || !dv)
    return fail(MSA_ERR_INVALID_ARG, "null pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(dO, 16) || !aligned(block_idx, 4) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16))
    return fail(MSA_ERR_INVALID_ARG, "misaligned pointer (q/k/v/o/dO/dq/dk/dv need 16 B)");
  const size_t need = msa_sparse_attn_bwd_workspace_min(N, H_q, H_kv, d_h, B_k, k_sel);
  if (!ws || ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes is below the minimum %zu", ws ? ws_bytes : 0, need);
  if (!aligned(ws, 256)) return fail(MSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const int64_t B = (N + B_k - 1) / B_k;
  uint8_t* w = static_cast<uint8_t*>(ws);
  float* D = reinterpret_cast<float*>(w);
  const size_t dbytes = bwd_d_bytes(N, H_q);
  const int64_t W = window_for_bytes(N, B, H_q, H_kv, k_sel, ws_bytes - dbytes, msa::kPartsBwd);
  const msa::AttnWorkspace L = msa::attn_workspace_layout(W, H_q, H_kv, k_sel, B, msa::kPartsBwd);
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  hipError_t e = msa::launch_bwd_prepare(static_cast<const uint16_t*>(dO), o, N * H_q, D, dk, dv,
                                         N * H_kv * msa::kHeadDim, stream);
  if (e != hipSuccess) return hip_fail(e, "backward prepare launch");
  const int cus = num_cus();
  for (int64_t w0 = 0; w0 < N; w0 += W) {
    const int64_t Wn = (N - w0 < W) ? N - w0 : W;
    e = msa::launch_bwd_window(static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                               static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dO), lse, D, block_idx,
                               N, B, B_k, H_q, H_kv, k_sel, scale, w0, Wn, cus, dq, dk, dv, w + dbytes, L, stream,
                               w0 == 0 ? clock_for(cus + 8) : nullptr);
    if (e != hipSuccess) return hip_fail(e, "backward launch");
  }
  return ok();
}

msa_status_t msa_set_profile_clock(uint64_t* clock, int64_t slots) {
  if (slots == 0) {
    g_clock = nullptr;
    g_clock_slots = 0;
    return ok();
  }
  if (slots < 0 || !clock || !aligned(clock, 8))
    return fail(MSA_ERR_INVALID_ARG, "msa_set_profile_clock takes a device buffer of slots >= 1 uint64");
  g_clock = clock;
  g_clock_slots = slots;
  return ok();
}

msa_status_t msa_set_profile_events(void* const* events, int n) {
  if (n == 0) {
    g_phase_windows = 0;
    return ok();
  }
  if (n < 0 || n % 4 != 0 || n > 4 * kMaxProfileWindows || !events)
    return fail(MSA_ERR_INVALID_ARG, "msa_set_profile_events takes 0 or 4 * m events, 1 <= m <= %d",
                kMaxProfileWindows);
  for (int i = 0; i < n; ++i)
    if (!events[i]) return fail(MSA_ERR_INVALID_ARG, "null event handle");
  for (int i = 0; i < n; ++i) g_phase_events[i] = static_cast<hipEvent_t>(events[i]);
  g_phase_windows = n / 4;
  return ok();
}

static msa_status_t check_decode_shape(int batch, int64_t max_len, int H_q, int H_kv, int d_h, int d_idx, int B_k,
                                       int k) {
  if (batch < 0) return fail(MSA_ERR_INVALID_ARG, "batch must be >= 0");
  if (max_len < 0) return fail(MSA_ERR_INVALID_ARG, "max_len must be >= 0");
  msa_status_t st = check_common(max_len, d_h, msa::kHeadDim, "d_h", B_k, k);
  if (st != MSA_OK) return st;
  if (d_idx != msa::kIndexDim) return fail(MSA_ERR_UNSUPPORTED, "d_idx must be 64 (got %d)", d_idx);
  if (H_kv < 1 || H_q < 1 || H_q % H_kv != 0)
    return fail(MSA_ERR_INVALID_ARG, "H_q must be a positive multiple of H_kv");
  if (H_kv > 16) return fail(MSA_ERR_UNSUPPORTED, "decode supports H_kv <= 16");
  const int G = H_q / H_kv;
  if (!is_pow2(G) || G > 16) return fail(MSA_ERR_UNSUPPORTED, "decode supports H_q / H_kv in {1,2,4,8,16}");
  return MSA_OK;
}

size_t msa_decode_workspace(int batch, int H_q, int H_kv, int d_h, int d_idx, int B_k, int k, int64_t max_len) {
  if (check_decode_shape(batch, max_len, H_q, H_kv, d_h, d_idx, B_k, k) != MSA_OK) return 0;
  const int64_t Bmax = (max_len + B_k - 1) / B_k;
  return msa::decode_workspace_layout(batch, H_q, H_kv, k, Bmax > 0 ? Bmax : 1).total;
}

// msa_decode after its shape checks: pointers, workspace, launch.
static msa_status_t decode_run(const void* q, const void* q_idx, const void* k_cache, const void* v_cache,
                               const void* k_idx_cache, const int64_t* cu_seqlens, int batch, int64_t T,
                               int64_t max_len,
                               int H_q, int H_kv, int B_k, int k, float scale, int32_t* block_idx, float* o,
                               float* lse, void* ws, size_t ws_bytes, void* hip_stream) {
  if (!q || !q_idx || !k_cache || !v_cache || !k_idx_cache || !cu_seqlens || !block_idx || !o || !lse)
    return fail(MSA_ERR_INVALID_ARG, "null pointer");
  if (!aligned(q, 16) || !aligned(q_idx, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(k_idx_cache, 16) || !aligned(cu_seqlens, 8) || !aligned(block_idx, 4) || !aligned(o, 16) ||
      !aligned(lse, 4))
    return fail(MSA_ERR_INVALID_ARG, "misaligned pointer");
  const size_t need = msa_decode_workspace(batch, H_q, H_kv, msa::kHeadDim, msa::kIndexDim, B_k, k, max_len);
  if (!ws || ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes is below the required %zu", ws ? ws_bytes : 0, need);
  if (!aligned(ws, 256)) return fail(MSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const int64_t Bmax = (max_len + B_k - 1) / B_k;
  const msa::DecodeWorkspace L = msa::decode_workspace_layout(batch, H_q, H_kv, k, Bmax);
  hipError_t e = msa::launch_decode(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(q_idx), static_cast<const uint16_t*>(k_cache),
      static_cast<const uint16_t*>(v_cache), static_cast<const uint16_t*>(k_idx_cache), cu_seqlens, batch, T, Bmax, B_k,
      H_q, H_kv, k, scale, block_idx, o, lse, static_cast<uint8_t*>(ws), L, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

msa_status_t msa_decode(const void* q, const void* q_idx, const void* k_cache, const void* v_cache,
                        const void* k_idx_cache, const int64_t* cu_seqlens, int batch, int64_t T, int64_t max_len,
                        int H_q, int H_kv, int d_h, int d_idx, int B_k, int k, float scale, int32_t* block_idx,
                        float* o, float* lse, void* ws, size_t ws_bytes, void* hip_stream) {
  msa_status_t st = check_decode_shape(batch, max_len, H_q, H_kv, d_h, d_idx, B_k, k);
  if (st != MSA_OK) return st;
  if (T < 0) return fail(MSA_ERR_INVALID_ARG, "T must be >= 0");
  if (!(scale > 0.f) || scale != scale) return fail(MSA_ERR_INVALID_ARG, "scale must be a positive number");
  if (batch == 0) return ok();
  if (max_len == 0) return fail(MSA_ERR_INVALID_ARG, "max_len must be >= 1 when batch > 0");
  return decode_run(q, q_idx, k_cache, v_cache, k_idx_cache, cu_seqlens, batch, T, max_len, H_q, H_kv, B_k, k,
                    scale, block_idx, o, lse, ws, ws_bytes, hip_stream);
}

msa_status_t msa_decode_noalloc(const void* q, const void* q_idx, const void* k_cache, const void* v_cache,
                                const void* k_idx_cache, const int64_t* cu_seqlens, int batch, int64_t T,
                                int64_t max_len, int H_q, int H_kv, int d_h, int d_idx, int B_k, int k, float scale,
                                int32_t* block_idx, float* o, float* lse, void* hip_stream) {
  msa_status_t st = check_decode_shape(batch, max_len, H_q, H_kv, d_h, d_idx, B_k, k);
  if (st != MSA_OK) return st;
  if (T < 0) return fail(MSA_ERR_INVALID_ARG, "T must be >= 0");
  if (!(scale > 0.f) || scale != scale) return fail(MSA_ERR_INVALID_ARG, "scale must be a positive number");
  if (batch == 0) return ok();
  if (max_len == 0) return fail(MSA_ERR_INVALID_ARG, "max_len must be >= 1 when batch > 0");
  const size_t need = msa_decode_workspace(batch, H_q, H_kv, d_h, d_idx, B_k, k, max_len);
  if (need > (size_t)MSA_DECODE_NOALLOC_SCRATCH_BYTES)
    return fail(MSA_ERR_WORKSPACE,
                "these shapes need %zu bytes of scratch, above the library's static %zu bytes; "
                "call msa_decode with a workspace instead", need, (size_t)MSA_DECODE_NOALLOC_SCRATCH_BYTES);
  uint8_t* ws = nullptr;
  if ((st = scratch_on_current_device(&ws)) != MSA_OK) return st;
  return decode_run(q, q_idx, k_cache, v_cache, k_idx_cache, cu_seqlens, batch, T, max_len, H_q, H_kv, B_k, k,
                    scale, block_idx, o, lse, ws, (size_t)MSA_DECODE_NOALLOC_SCRATCH_BYTES, hip_stream);
}

msa_status_t msa_decode_paged(const void* q, const void* q_idx, const void* k_pages, const void* v_pages,
                              float k_scale, float v_scale, const void* k_idx_pages, const int32_t* block_table,
                              int64_t max_blocks, int64_t num_pages, const int64_t* seqlens, int batch,
                              int64_t max_len, int H_q,
                              int H_kv, int d_h, int d_idx, int B_k, int k, float scale, int32_t* block_idx,
                              float* o, float* lse, void* ws, size_t ws_bytes, void* hip_stream) {
  msa_status_t st = check_decode_shape(batch, max_len, H_q, H_kv, d_h, d_idx, B_k, k);
  if (st != MSA_OK) return st;
  if (!(scale > 0.f) || scale != scale) return fail(MSA_ERR_INVALID_ARG, "scale must be a positive number");
  if (!(k_scale > 0.f) || !(v_scale > 0.f) || k_scale != k_scale || v_scale != v_scale ||
      k_scale == __builtin_inff() || v_scale == __builtin_inff())
    return fail(MSA_ERR_INVALID_ARG, "k_scale and v_scale must be positive finite numbers");
  if (batch == 0) return ok();
  if (max_len == 0) return fail(MSA_ERR_INVALID_ARG, "max_len must be >= 1 when batch > 0");
  const int64_t Bmax = (max_len + B_k - 1) / B_k;
  if (max_blocks < Bmax)
    return fail(MSA_ERR_INVALID_ARG, "max_blocks (%lld) must cover ceil(max_len / B_k) = %lld",
                (long long)max_blocks, (long long)Bmax);
  if (num_pages < 1) return fail(MSA_ERR_INVALID_ARG, "num_pages must be >= 1 when batch > 0");
  if (!q || !q_idx || !k_pages || !v_pages || !k_idx_pages || !block_table || !seqlens || !block_idx || !o || !lse)
    return fail(MSA_ERR_INVALID_ARG, "null pointer");
  if (!aligned(q, 16) || !aligned(q_idx, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) ||
      !aligned(k_idx_pages, 16) || !aligned(block_table, 4) || !aligned(seqlens, 8) || !aligned(block_idx, 4) ||
      !aligned(o, 16) || !aligned(lse, 4))
    return fail(MSA_ERR_INVALID_ARG, "misaligned pointer");
  const size_t need = msa_decode_workspace(batch, H_q, H_kv, d_h, d_idx, B_k, k, max_len);
  if (!ws || ws_bytes < need)
    return fail(MSA_ERR_WORKSPACE, "workspace of %zu bytes is below the required %zu", ws ? ws_bytes : 0, need);
  if (!aligned(ws, 256)) return fail(MSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  const msa::DecodeWorkspace L = msa::decode_workspace_layout(batch, H_q, H_kv, k, Bmax);
  hipError_t e = msa::launch_decode_paged(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(q_idx), static_cast<const uint8_t*>(k_pages),
      static_cast<const uint8_t*>(v_pages), k_scale, v_scale, static_cast<const uint16_t*>(k_idx_pages), block_table,
      max_blocks, num_pages, seqlens, batch, Bmax, B_k, H_q, H_kv, k, scale, block_idx, o, lse,
      static_cast<uint8_t*>(ws), L, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "paged decode launch");
  return ok();
}

}  // extern "C"
