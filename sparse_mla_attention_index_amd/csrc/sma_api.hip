// C ABI of the sparse-MLA prefill library: argument validation, workspace
// carving and kernel dispatch on the caller's stream.  Declarations and the
// contract of every entry point are in include/sma.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/sma.h"
#include "sma_launch.h"

// Scratch of sma_dcp_shard_partial_noalloc (its callers cannot allocate):
// the rank's local index list and the row slices' partials.
constexpr size_t kStaticScratchBytes = SMA_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

// Debug builds (SMA_DEBUG_CHECKS=1, libsma_debug.so): index lists and query
// positions held in device memory are scanned before the launch that reads
// them, and a value a release build would skip or clamp is reported as an
// error; workspace is filled with 0xFF bytes (fp32 NaN) before use.
#ifndef SMA_DEBUG_CHECKS
#define SMA_DEBUG_CHECKS 0
#endif
#if SMA_DEBUG_CHECKS
// index of the first out-of-range element the last check on this device found
static __device__ unsigned long long dbg_first_bad;
#endif

namespace {

thread_local std::string g_err;

sma_status fail(sma_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
sma_status fail(sma_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

sma_status hip_fail(hipError_t e, const char* what) {
  return fail(SMA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxDevices = 64;
// Per-device facts queried once: 0 = not yet known.  Concurrent first calls
// may both query; they store the same value, and the atomics make that a
// well-defined race.
std::atomic<int> g_dev_ok[kMaxDevices];   // 1 gfx950, -1 other
std::atomic<int> g_dev_cus[kMaxDevices];  // compute units

sma_status check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SMA_ERR_UNSUPPORTED, "device ordinal %d", dev);
  int ok = g_dev_ok[dev].load(std::memory_order_relaxed);
  if (ok == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
    ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
    g_dev_ok[dev].store(ok, std::memory_order_relaxed);
  }
  if (ok != 1) return fail(SMA_ERR_UNSUPPORTED, "device %d is not gfx950", dev);
  return SMA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int64_t kMaxKeys = 0x7FFFFFFFLL;
constexpr int32_t kMinScoreBlock = 64;   // query rows of scores the prefill workspace must hold

#define SMA_CHECK(cond, ...) \
  do {                       \
    if (!(cond)) return fail(SMA_ERR_INVALID_ARG, __VA_ARGS__); \
  } while (0)

#if SMA_DEBUG_CHECKS
__global__ void dbg_reset_kernel(unsigned long long* first_bad) { *first_bad = ~0ull; }

__global__ void dbg_range_kernel(const int32_t* v, int64_t n, int32_t lo, int32_t hi,
                                 unsigned long long* first_bad) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += step) {
    const int32_t x = v[i];
    if (x < lo || x > hi) atomicMin(first_bad, (unsigned long long)i);
  }
}

// Reports the first of v[0 .. n) outside [lo, hi] as SMA_ERR_INVALID_ARG.
// Synchronises `st` (debug builds only).
sma_status dbg_range(const int32_t* v, int64_t n, int32_t lo, int32_t hi, const char* what, hipStream_t st) {
  if (n <= 0) return SMA_OK;
  void* addr = nullptr;
  hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(dbg_first_bad));
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(dbg_first_bad)");
  auto* first_bad = static_cast<unsigned long long*>(addr);
  hipLaunchKernelGGL(dbg_reset_kernel, dim3(1), dim3(1), 0, st, first_bad);
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 8192);
  hipLaunchKernelGGL(dbg_range_kernel, dim3((unsigned)blocks), dim3(256), 0, st, v, n, lo, hi, first_bad);
  unsigned long long first = 0;
  e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpyAsync(&first, first_bad, sizeof first, hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "debug range check");
  if (first == ~0ull) return SMA_OK;
  int32_t val = 0;
  e = hipMemcpy(&val, v + first, sizeof val, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e, "debug range check");
  return fail(SMA_ERR_INVALID_ARG, "debug check: %s[%llu] = %d outside [%d, %d]", what, first, (int)val, (int)lo,
              (int)hi);
}

sma_status dbg_poison(void* ws, size_t bytes, hipStream_t st) {
  if (ws == nullptr || bytes == 0) return SMA_OK;
  hipError_t e = hipMemsetAsync(ws, 0xFF, bytes, st);
  return e == hipSuccess ? SMA_OK : hip_fail(e, "debug workspace fill");
}

#define SMA_DEBUG_RANGE(v, n, lo, hi, what, st)                       \
  do {                                                                \
    const sma_status dbg_s = dbg_range(v, n, lo, hi, what, st);       \
    if (dbg_s != SMA_OK) return dbg_s;                                \
  } while (0)
#define SMA_DEBUG_POISON(ws, bytes, st)                               \
  do {                                                                \
    const sma_status dbg_s = dbg_poison(ws, bytes, st);               \
    if (dbg_s != SMA_OK) return dbg_s;                                \
  } while (0)
#else
#define SMA_DEBUG_RANGE(v, n, lo, hi, what, st) \
  do {                                          \
  } while (0)
#define SMA_DEBUG_POISON(ws, bytes, st) \
  do {                                  \
  } while (0)
#endif

sma_status validate_indexer(const void* q_idx, const float* w, int64_t w_stride, const void* k_idx,
                            const float* k_scale, int32_t k_dtype, const int32_t* q_pos, int32_t n_q,
                            int64_t n_k, int32_t h_idx, int32_t d_idx, bool pos_from_caller = true) {
  SMA_CHECK(n_q >= 0, "n_q = %d < 0", n_q);
  SMA_CHECK(n_k >= 1 && n_k <= kMaxKeys, "n_k = %lld out of [1, 2^31)", (long long)n_k);
  if (!(h_idx == 8 || h_idx == 16 || h_idx == 32 || h_idx == 64))
    return fail(SMA_ERR_UNSUPPORTED, "h_idx = %d (supported: 8, 16, 32, 64)", h_idx);
  if (!(d_idx == 64 || d_idx == 128))
    return fail(SMA_ERR_UNSUPPORTED, "d_idx = %d (supported: 64, 128)", d_idx);
  SMA_CHECK(k_dtype == SMA_DT_BF16 || k_dtype == SMA_DT_FP8_E4M3, "k_dtype = %d", k_dtype);
  SMA_CHECK(k_idx != nullptr, "k_idx is NULL");
  SMA_CHECK((k_dtype == SMA_DT_FP8_E4M3) == (k_scale != nullptr),
            "k_scale must be given exactly when the keys are FP8");
  SMA_CHECK(aligned(k_idx, 16), "k_idx not 16-byte aligned");
  SMA_CHECK(w_stride == 0 || w_stride >= h_idx, "w_stride = %lld (0 or >= h_idx)", (long long)w_stride);
  if (n_q > 0) {
    SMA_CHECK(q_idx && w && (q_pos || !pos_from_caller), "q_idx, w and q_pos must be non-NULL");
    SMA_CHECK(aligned(q_idx, 16), "q_idx not 16-byte aligned");
  }
  return SMA_OK;
}

// FP8 queries: FP8 keys, the 64 x 128 shape, one scale per (query, head).
sma_status validate_indexer_fp8(const uint8_t* q_idx, const float* q_scale, const float* w, int64_t w_stride,
                                const uint8_t* k_idx, const float* k_scale, const int32_t* q_pos, int32_t n_q,
                                int64_t n_k, int32_t h_idx, int32_t d_idx) {
  sma_status s = validate_indexer(q_idx, w, w_stride, k_idx, k_scale, SMA_DT_FP8_E4M3, q_pos, n_q, n_k, h_idx,
                                  d_idx);
  if (s != SMA_OK) return s;
  SMA_CHECK(k_scale != nullptr && aligned(k_scale, 4), "k_scale is NULL or not 4-byte aligned");
  if (h_idx != 64 || d_idx != 128)
    return fail(SMA_ERR_UNSUPPORTED, "FP8 queries: h_idx = %d, d_idx = %d (supported: 64 x 128)", h_idx, d_idx);
  if (n_q > 0) SMA_CHECK(q_scale != nullptr, "q_scale is NULL");
  return SMA_OK;
}

sma_status validate_topk(int32_t n_q, int64_t n_k, int32_t top_k) {
  SMA_CHECK(n_q >= 0, "n_q = %d < 0", n_q);
  SMA_CHECK(n_k >= 1 && n_k <= kMaxKeys, "n_k = %lld out of [1, 2^31)", (long long)n_k);
  SMA_CHECK(top_k >= 1 && top_k <= SMA_MAX_TOPK, "top_k = %d out of [1, %d]", top_k, SMA_MAX_TOPK);
  return SMA_OK;
}

sma_status validate_mla(const uint16_t* q, const void* kv, const float* kv_scale, int32_t kv_dtype,
                        int64_t n_k, const int32_t* idx, int32_t n_q, int32_t top_k, float sm_scale,
                        void* out, int32_t out_dtype, bool idx_may_be_null) {
  SMA_CHECK(n_q >= 0, "n_q = %d < 0", n_q);
  SMA_CHECK(n_k >= 1 && n_k <= kMaxKeys, "n_k = %lld out of [1, 2^31)", (long long)n_k);
  SMA_CHECK(top_k >= 1 && top_k <= SMA_MAX_TOPK, "top_k = %d out of [1, %d]", top_k, SMA_MAX_TOPK);
  SMA_CHECK(kv_dtype == SMA_DT_BF16 || kv_dtype == SMA_DT_FP8_E4M3 || kv_dtype == SMA_DT_FP8_DS_MLA,
            "kv_dtype = %d", kv_dtype);
  SMA_CHECK(out_dtype == SMA_DT_BF16 || out_dtype == SMA_DT_FP32, "out_dtype = %d", out_dtype);
  SMA_CHECK(kv != nullptr, "kv is NULL");
  SMA_CHECK((kv_dtype == SMA_DT_FP8_E4M3) == (kv_scale != nullptr),   // fp8_ds_mla rows carry their scales
            "kv_scale must be given exactly when the KV is FP8");
  SMA_CHECK(aligned(kv, 16), "kv not 16-byte aligned");
  SMA_CHECK(std::isfinite(sm_scale) && sm_scale > 0.f, "sm_scale = %g (finite and > 0)", (double)sm_scale);
  if (n_q > 0) {
    SMA_CHECK(q && out && (idx || idx_may_be_null), "q, idx and out must be non-NULL");
    SMA_CHECK(aligned(q, 16), "q not 16-byte aligned");
    SMA_CHECK(aligned(out, out_dtype == SMA_DT_FP32 ? 16 : 8), "out not aligned");
  }
  return SMA_OK;
}

sma::IdxArgs idx_args(const void* q_idx, const float* q_scale, const float* w, int64_t w_stride,
                      const void* k_idx, const float* k_scale, int32_t k_dtype, const int32_t* q_pos,
                      int32_t n_q, int64_t n_k, int32_t h_idx, int32_t d_idx, float* scores, int64_t ld) {
  sma::IdxArgs a;
  a.q_idx = q_idx; a.q_scale = q_scale; a.w = w; a.w_stride = w_stride; a.k_idx = k_idx; a.k_scale = k_scale;
  a.fp8 = k_dtype == SMA_DT_FP8_E4M3; a.q_pos = q_pos; a.n_q = n_q; a.n_k = n_k;
  a.h_idx = h_idx; a.d_idx = d_idx; a.scores = scores; a.ld = ld;
  return a;
}

// Workspace of one block of qb query rows in the composed path: their scores
// plus, for rows longer than the on-chip top-k holds, the split top-k's
// buffers.
size_t score_block_bytes(int64_t qb, int64_t n_k, int32_t top_k) {
  size_t b = align_up((size_t)qb * (size_t)n_k * 4, 256);
  if (sma::topk_long_wanted(n_k)) b += align_up(sma::topk_long_bytes((int32_t)qb, n_k, top_k), 256);
  return b;
}

size_t prefill_fixed_bytes(int32_t n_q, int32_t top_k, bool need_idx, bool need_pos) {
  size_t b = 0;
  if (need_pos) b += align_up((size_t)n_q * 4, 256);
  if (need_idx) b += align_up((size_t)n_q * top_k * 4, 256);
  return b;
}

// The composed path shared by sma_prefill and sma_pcp_rank_share.  `pos` is
// a device array of n_q positions; `ws` past `fixed` holds score blocks.
sma_status run_prefill(const void* q_idx, const float* q_scale, const float* w, int64_t w_stride,
                       const void* k_idx,
                       const float* k_scale, int32_t k_dtype, const uint16_t* q, const void* kv,
                       const float* kv_scale, int32_t kv_dtype, const int32_t* pos, int32_t n_q,
                       int64_t n_k, int32_t h_idx, int32_t d_idx, int32_t top_k, float sm_scale,
                       void* out, int32_t out_dtype, float* lse, int32_t* idx, uint8_t* score_ws,
                       size_t score_ws_bytes, hipStream_t st) {
  // the largest block of query rows whose scores and top-k buffers fit (the
  // size grows with the rows), rounded down to a multiple of 16 when it
  // holds 16 or more but not all of them
  int64_t lo = 0, hi = n_q;
  while (lo < hi) {
    const int64_t mid = lo + (hi - lo + 1) / 2;
    if (score_block_bytes(mid, n_k, top_k) <= score_ws_bytes) lo = mid;
    else hi = mid - 1;
  }
  int64_t qb = lo;
  if (qb < n_q && qb >= 16) qb = qb / 16 * 16;
  if (qb < 1) return fail(SMA_ERR_WORKSPACE, "workspace holds no score block");
  float* scores = reinterpret_cast<float*>(score_ws);
  uint8_t* topk_ws = score_ws + align_up((size_t)qb * (size_t)n_k * 4, 256);
  const size_t topk_ws_bytes = score_ws_bytes - align_up((size_t)qb * (size_t)n_k * 4, 256);
  for (int64_t q0 = 0; q0 < n_q; q0 += qb) {
    const int32_t nb = (int32_t)((n_q - q0) < qb ? (n_q - q0) : qb);
    // bf16 query rows take 2 bytes an element, FP8 ones 1 plus a scale per head
    const size_t q_row_bytes = (size_t)h_idx * d_idx * (q_scale ? 1 : 2);
    sma::IdxArgs ia = idx_args(static_cast<const uint8_t*>(q_idx) + q0 * q_row_bytes,
                               q_scale ? q_scale + q0 * h_idx : nullptr, w + q0 * w_stride, w_stride, k_idx,
                               k_scale, k_dtype, pos + q0, nb, n_k, h_idx, d_idx, scores, n_k);
    hipError_t e = sma::launch_index_scores(ia, st);
    if (e != hipSuccess) return hip_fail(e, "index_scores launch");
    sma::TopkArgs ta{scores, n_k, pos + q0, nb, n_k, top_k, idx + q0 * top_k, topk_ws, topk_ws_bytes};
    e = sma::launch_topk(ta, st);
    if (e != hipSuccess) return hip_fail(e, "topk launch");
  }
  // the score blocks are dead once the index lists exist: their space holds
  // the attention kernel's split partials for small batches
  sma::MlaArgs ma{q, kv, kv_scale, kv_dtype != SMA_DT_BF16, n_k, idx, n_q, top_k, sm_scale,
                  out, out_dtype == SMA_DT_FP32, lse, score_ws, score_ws_bytes};
  ma.ds_mla = kv_dtype == SMA_DT_FP8_DS_MLA;
  hipError_t e = sma::launch_sparse_mla(ma, st);
  if (e != hipSuccess) return hip_fail(e, "sparse_mla launch");
  return SMA_OK;
}


// sma_prefill and sma_prefill_fp8_indexer after their indexer checks.
sma_status prefill_entry(const void* q_idx, const float* q_scale, const float* w, int64_t w_stride,
                         const void* k_idx, const float* k_scale, int32_t k_dtype, const uint16_t* q,
                         const void* kv, const float* kv_scale, int32_t kv_dtype, const int32_t* q_pos,
                         int32_t n_q, int64_t n_k, int32_t h_idx, int32_t d_idx, int32_t top_k, float sm_scale,
                         void* out, int32_t out_dtype, float* lse, int32_t* idx_out, void* ws, size_t ws_bytes,
                         void* stream) {
  sma_status s = validate_mla(q, kv, kv_scale, kv_dtype, n_k, idx_out, n_q, top_k, sm_scale, out, out_dtype, true);
  if (s != SMA_OK) return s;
  if (n_q == 0) return SMA_OK;
  const size_t fixed = prefill_fixed_bytes(n_q, top_k, idx_out == nullptr, false);
  const int32_t blk = n_q < kMinScoreBlock ? n_q : kMinScoreBlock;
  const size_t need = fixed + score_block_bytes(blk, n_k, top_k);
  if (ws_bytes < need || (ws == nullptr && need > 0))
    return fail(SMA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  SMA_CHECK(aligned(ws, 256), "workspace not 256-byte aligned");
  if ((s = check_device()) != SMA_OK) return s;
  SMA_DEBUG_RANGE(q_pos, n_q, -1, (int32_t)(n_k - 1), "q_pos", (hipStream_t)stream);
  SMA_DEBUG_POISON(ws, ws_bytes, (hipStream_t)stream);
  uint8_t* p = static_cast<uint8_t*>(ws);
  int32_t* idx = idx_out;
  if (!idx) {
    idx = reinterpret_cast<int32_t*>(p);
    p += align_up((size_t)n_q * top_k * 4, 256);
  }
  return run_prefill(q_idx, q_scale, w, w_stride, k_idx, k_scale, k_dtype, q, kv, kv_scale, kv_dtype, q_pos,
                     n_q, n_k, h_idx, d_idx, top_k, sm_scale, out, out_dtype, lse, idx, p,
                     ws_bytes - (size_t)(p - static_cast<uint8_t*>(ws)), (hipStream_t)stream);
}

sma_status validate_dcp(int32_t rank, int32_t dcp_size, const uint16_t* q, const void* kv_local,
                        const float* kv_scale_local, int32_t kv_dtype, int64_t n_k_local, const int32_t* idx,
                        int32_t n_q, int32_t top_k, float sm_scale, float* out_partial, float* lse_partial) {
  SMA_CHECK(dcp_size >= 1, "dcp_size = %d < 1", dcp_size);
  SMA_CHECK(rank >= 0 && rank < dcp_size, "rank = %d not in [0, %d)", rank, dcp_size);
  sma_status s = validate_mla(q, kv_local, kv_scale_local, kv_dtype, n_k_local, idx, n_q, top_k, sm_scale,
                              out_partial, SMA_DT_FP32, false);
  if (s != SMA_OK) return s;
  if (n_q > 0) SMA_CHECK(lse_partial != nullptr, "lse_partial is NULL");
  return SMA_OK;
}

// One DCP rank's partial after validation: the rank's local index list at the
// start of `ws`, the row slices' partials in the rest.
sma_status run_dcp_partial(int32_t rank, int32_t dcp_size, const uint16_t* q, const void* kv_local,
                           const float* kv_scale_local, int32_t kv_dtype, int64_t n_k_local, const int32_t* idx,
                           int32_t n_q, int32_t top_k, float sm_scale, float* out_partial, float* lse_partial,
                           uint8_t* ws, size_t ws_bytes, hipStream_t st) {
  const size_t idx_bytes = align_up((size_t)n_q * (size_t)top_k * 4, 256);
  int32_t* local = reinterpret_cast<int32_t*>(ws);
  hipError_t e = sma::launch_dcp_local_idx(idx, n_q, top_k, rank, dcp_size, n_k_local, local, st);
  if (e != hipSuccess) return hip_fail(e, "dcp_local_idx launch");
  sma::MlaArgs a{q, kv_local, kv_scale_local, kv_dtype != SMA_DT_BF16, n_k_local, local, n_q, top_k,
                 sm_scale, out_partial, true, lse_partial, ws + idx_bytes, ws_bytes - idx_bytes};
  a.ds_mla = kv_dtype == SMA_DT_FP8_DS_MLA;
  e = sma::launch_sparse_mla(a, st);
  return e == hipSuccess ? SMA_OK : hip_fail(e, "sparse_mla launch");
}

// The no-allocation entry's scratch: one static device array per device,
// reached through the address hipGetSymbolAddress returns for the current
// device (the array's name is only a host-side stand-in).  Taken once per
// device, under a lock, at that device's first call; kept until the process
// ends.
std::atomic<uint8_t*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

sma_status static_scratch(uint8_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(SMA_ERR_UNSUPPORTED, "device ordinal %d", dev);
  uint8_t* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
      if (addr == nullptr) return fail(SMA_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
      p = static_cast<uint8_t*>(addr);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SMA_OK;
}

}  // namespace

extern "C" {

sma_status sma_index_scores(const uint16_t* q_idx, const float* w, int64_t w_stride, const void* k_idx,
                            const float* k_scale, int32_t k_dtype, const int32_t* q_pos, int32_t n_q,
                            int64_t n_k, int32_t h_idx, int32_t d_idx, float* scores, int64_t ld_scores,
                            void* stream) {
  g_err.clear();
  sma_status s = validate_indexer(q_idx, w, w_stride, k_idx, k_scale, k_dtype, q_pos, n_q, n_k, h_idx, d_idx);
  if (s != SMA_OK) return s;
  SMA_CHECK(ld_scores >= n_k, "ld_scores = %lld < n_k = %lld", (long long)ld_scores, (long long)n_k);
  if (n_q > 0) SMA_CHECK(scores != nullptr, "scores is NULL");
  if (n_q == 0) return SMA_OK;
  if ((s = check_device()) != SMA_OK) return s;
  SMA_DEBUG_RANGE(q_pos, n_q, -1, (int32_t)(n_k - 1), "q_pos", (hipStream_t)stream);
  hipError_t e = sma::launch_index_scores(
      idx_args(q_idx, nullptr, w, w_stride, k_idx, k_scale, k_dtype, q_pos, n_q, n_k, h_idx, d_idx, scores,
               ld_scores),
      (hipStream_t)stream);
  return e == hipSuccess ? SMA_OK : hip_fail(e, "index_scores launch");
}

sma_status sma_index_scores_fp8(const uint8_t* q_idx, const float* q_scale, const float* w, int64_t w_stride,
                                const uint8_t* k_idx, const float* k_scale, const int32_t* q_pos, int32_t n_q,
                                int64_t n_k, int32_t h_idx, int32_t d_idx, float* scores, int64_t ld_scores,
                                void* stream) {
  g_err.clear();
  sma_status s = validate_indexer_fp8(q_idx, q_scale, w, w_stride, k_idx, k_scale, q_pos, n_q, n_k, h_idx, d_idx);
  if (s != SMA_OK) return s;
  SMA_CHECK(ld_scores >= n_k, "ld_scores = %lld < n_k = %lld", (long long)ld_scores, (long long)n_k);
  if (n_q > 0) SMA_CHECK(scores != nullptr, "scores is NULL");
  if (n_q == 0) return SMA_OK;
  if ((s = check_device()) != SMA_OK) return s;
  SMA_DEBUG_RANGE(q_pos, n_q, -1, (int32_t)(n_k - 1), "q_pos", (hipStream_t)stream);
  hipError_t e = sma::launch_index_scores(idx_args(q_idx, q_scale, w, w_stride, k_idx, k_scale, SMA_DT_FP8_E4M3,
                                                   q_pos, n_q, n_k, h_idx, d_idx, scores, ld_scores),
                                          (hipStream_t)stream);
  return e == hipSuccess ? SMA_OK : hip_fail(e, "index_scores_fp8 launch");
}

sma_status sma_quantize_fp8_rows(const uint16_t* x, int64_t n_rows, int32_t d, uint8_t* codes, float* scale,
                                 void* stream) {
  g_err.clear();
  SMA_CHECK(n_rows >= 0 && n_rows <= ((int64_t)1 << 36), "n_rows = %lld out of [0, 2^36]", (long long)n_rows);
  if (d != 64 && d != 128) return fail(SMA_ERR_UNSUPPORTED, "d = %d (supported: 64, 128)", d);
  if (n_rows == 0) return SMA_OK;
  SMA_CHECK(x && codes && scale, "x, codes and scale must be non-NULL");
  SMA_CHECK(aligned(x, 16), "x not 16-byte aligned");
  SMA_CHECK(aligned(codes, 8), "codes not 8-byte aligned");
  SMA_CHECK(aligned(scale, 4), "scale not 4-byte aligned");
  sma_status s = check_device();
  if (s != SMA_OK) return s;
  hipError_t e = sma::launch_quantize_fp8_rows(x, n_rows, d, codes, scale, (hipStream_t)stream);
  return e == hipSuccess ? SMA_OK : hip_fail(e, "quantize_fp8_rows launch");
}

sma_status sma_absorb_q(const uint16_t* q_nope, const uint16_t* w_uk, int32_t n, int32_t heads, uint16_t* q_out,
                        int64_t ld_out, void* stream) {
  g_err.clear();
  SMA_CHECK(n >= 0, "n = %d < 0", n);
  SMA_CHECK(heads >= 1 && heads <= 1024, "heads = %d out of [1, 1024]", heads);
  SMA_CHECK(ld_out >= 512 && ld_out % 8 == 0, "ld_out = %lld (>= 512, a multiple of 8)", (long long)ld_out);
  if (n == 0) return SMA_OK;
  SMA_CHECK(q_nope && w_uk && q_out, "q_nope, w_uk and q_out must be non-NULL");
  SMA_CHECK(aligned(q_nope, 16) && aligned(w_uk, 16) && aligned(q_out, 16), "tensors must be 16-byte aligned");
  sma_status s = check_device();
  if (s != SMA_OK) return s;
  sma::BmmArgs a{q_nope, (int64_t)heads * 128, 128, w_uk, 512, 128 * 512, true,
                 q_out, (int64_t)heads * ld_out, ld_out, n, 512, 128, heads};
  hipError_t e = sma::launch_bmm_bf16(a, (hipStream_t)stream);
  return e == hipSuccess ? SMA_OK : hip_fail(e, "absorb_q launch");
}

sma_status sma_project_out(const uint16_t* o_lat, const uint16_t* w_uv, int32_t n, int32_t heads, uint16_t* out,
                           void* stream) {
  g_err.clear();
  SMA_CHECK(n >= 0, "n = %d < 0", n);
  SMA_CHECK(heads >= 1 && heads <= 1024, "heads = %d out of [1, 1024]", heads);
  if (n == 0) return SMA_OK;
  SMA_CHECK(o_lat && w_uv && out, "o_lat, w_uv and out must be non-NULL");
  SMA_CHECK(aligned(o_lat, 16) && aligned(w_uv, 16) && aligned(out, 16), "tensors must be 16-byte aligned");
  sma_status s = check_device();
  if (s != SMA_OK) return s;
  sma::BmmArgs a{o_lat, (int64_t)heads * 512, 512, w_uv, 512, 128 * 512, false,
                 out, (int64_t)heads * 128, 128, n, 128, 512, heads};
  hipError_t e = sma::launch_bmm_bf16(a, (hipStream_t)stream);
  return e == hipSuccess ? SMA_OK : hip_fail(e, "project_out launch");
}

sma_status sma_topk_select(const float* scores, int64_t ld_scores, const int32_t* q_pos, int32_t n_q,
                           int64_t n_k, int32_t top_k, int32_t* idx, void* ws, size_t ws_bytes,
                           void* stream) {
  g_err.clear();
  sma_status s = validate_topk(n_q, n_k, top_k);
  if (s != SMA_OK) return s;
  SMA_CHECK(ld_scores >= n_k, "ld_scores = %lld < n_k = %lld", (long long)ld_scores, (long long)n_k);
  if (n_q > 0) SMA_CHECK(scores && q_pos && idx, "scores, q_pos and idx must be non-NULL");
  if (n_q == 0) return SMA_OK;
  if (ws) SMA_CHECK(aligned(ws, 256), "workspace not 256-byte aligned");
  if ((s = check_device()) != SMA_OK) return s;
  SMA_DEBUG_RANGE(q_pos, n_q, -1, (int32_t)(n_k - 1), "q_pos", (hipStream_t)stream);
  SMA_DEBUG_POISON(ws, ws_bytes, (hipStream_t)stream);
  sma::TopkArgs a{scores, ld_scores, q_pos, n_q, n_k, top_k, idx, ws, ws ? ws_bytes : 0};
  hipError_t e = sma::launch_topk(a, (hipStream_t)stream);
  return e == hipSuccess ? SMA_OK : hip_fail(e, "topk launch");
}

sma_status sma_sparse_mla_prefill(const uint16_t* q, const void* kv, const float* kv_scale,
                                  int32_t kv_dtype, int64_t n_k, const int32_t* idx, int32_t n_q,
                                  int32_t top_k, float sm_scale, void* out, int32_t out_dtype,
                                  float* lse, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  sma_status s = validate_mla(q, kv, kv_scale, kv_dtype, n_k, idx, n_q, top_k, sm_scale, out,
                              out_dtype, false);
  if (s != SMA_OK) return s;
  if (n_q == 0) return SMA_OK;
  if ((s = check_device()) != SMA_OK) return s;
  if (ws && !aligned(ws, 256)) return fail(SMA_ERR_INVALID_ARG, "workspace not 256-byte aligned");
  SMA_DEBUG_RANGE(idx, (int64_t)n_q * top_k, -1, (int32_t)(n_k - 1), "idx", (hipStream_t)stream);
  SMA_DEBUG_POISON(ws, ws_bytes, (hipStream_t)stream);
  sma::MlaArgs a{q, kv, kv_scale, kv_dtype != SMA_DT_BF16, n_k, idx, n_q, top_k, sm_scale,
                 out, out_dtype == SMA_DT_FP32, lse, ws, ws ? ws_bytes : 0};
  a.ds_mla = kv_dtype == SMA_DT_FP8_DS_MLA;
  hipError_t e = sma::launch_sparse_mla(a, (hipStream_t)stream);
  return e == hipSuccess ? SMA_OK : hip_fail(e, "sparse_mla launch");
}

sma_status sma_dense_mha_prefill(const uint16_t* q, const uint16_t* kv, const uint16_t* w_uk, const uint16_t* w_uv,
                                 const int32_t* q_pos, int32_t n_q, int64_t n_k, float sm_scale, void* out,
                                 int32_t out_dtype, float* lse, void* ws, size_t ws_bytes, void* stream) {
  g_err.clear();
  SMA_CHECK(n_q >= 0, "n_q = %d < 0", n_q);
  SMA_CHECK(n_k >= 1 && n_k <= kMaxKeys, "n_k = %lld out of [1, 2^31)", (long long)n_k);
  SMA_CHECK(out_dtype == SMA_DT_BF16 || out_dtype == SMA_DT_FP32, "out_dtype = %d", out_dtype);
  SMA_CHECK(std::isfinite(sm_scale) && sm_scale > 0.f, "sm_scale = %g (finite and > 0)", (double)sm_scale);
  SMA_CHECK(kv && w_uk && w_uv, "kv, w_uk and w_uv must be non-NULL");
  SMA_CHECK(aligned(kv, 16) && aligned(w_uk, 16) && aligned(w_uv, 16), "kv, w_uk and w_uv must be 16-byte aligned");
  if (n_q == 0) return SMA_OK;
  SMA_CHECK(q && q_pos && out, "q, q_pos and out must be non-NULL");
  SMA_CHECK(aligned(q, 16) && aligned(out, 16), "q and out must be 16-byte aligned");
  SMA_CHECK((int64_t)n_q <= ((int64_t)1 << 31) / SMA_HEADS, "n_q = %d too large", n_q);
  const size_t need = sma::dense_mha_ws_bytes(n_k);
  if (ws == nullptr || ws_bytes < need)
    return fail(SMA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws ? ws_bytes : 0, need);
  SMA_CHECK(aligned(ws, 256), "workspace not 256-byte aligned");
  sma_status s = check_device();
  if (s != SMA_OK) return s;
  SMA_DEBUG_RANGE(q_pos, n_q, -1, (int32_t)(n_k - 1), "q_pos", (hipStream_t)stream);
  SMA_DEBUG_POISON(ws, ws_bytes, (hipStream_t)stream);
  sma::DenseMhaArgs a{q, kv, w_uk, w_uv, q_pos, n_q, n_k, sm_scale, out, out_dtype == SMA_DT_FP32, lse, ws};
  hipError_t e = sma::launch_dense_mha(a, (hipStream_t)stream);
  return e == hipSuccess ? SMA_OK : hip_fail(e, "dense_mha launch");
}

sma_status sma_dcp_shard_partial(int32_t rank, int32_t dcp_size, const uint16_t* q, const void* kv_local,
                                 const float* kv_scale_local, int32_t kv_dtype, int64_t n_k_local,
                                 const int32_t* idx, int32_t n_q, int32_t top_k, float sm_scale,
                                 float* out_partial, float* lse_partial, void* ws, size_t ws_bytes,
                                 void* stream) {
  g_err.clear();
  sma_status s = validate_dcp(rank, dcp_size, q, kv_local, kv_scale_local, kv_dtype, n_k_local, idx, n_q, top_k,
                              sm_scale, out_partial, lse_partial);
  if (s != SMA_OK || n_q == 0) return s;
  const size_t idx_bytes = align_up((size_t)n_q * (size_t)top_k * 4, 256);
  if (ws == nullptr || ws_bytes < idx_bytes)
    return fail(SMA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws ? ws_bytes : 0, idx_bytes);
  SMA_CHECK(aligned(ws, 256), "workspace not 256-byte aligned");
  if ((s = check_device()) != SMA_OK) return s;
  SMA_DEBUG_RANGE(idx, (int64_t)n_q * top_k, -1, INT32_MAX, "idx", (hipStream_t)stream);
  SMA_DEBUG_POISON(ws, ws_bytes, (hipStream_t)stream);
  return run_dcp_partial(rank, dcp_size, q, kv_local, kv_scale_local, kv_dtype, n_k_local, idx, n_q, top_k,
                         sm_scale, out_partial, lse_partial, static_cast<uint8_t*>(ws), ws_bytes,
                         (hipStream_t)stream);
}

sma_status sma_dcp_shard_partial_noalloc(int32_t rank, int32_t dcp_size, const uint16_t* q, const void* kv_local,
                                         const float* kv_scale_local, int32_t kv_dtype, int64_t n_k_local,
                                         const int32_t* idx, int32_t n_q, int32_t top_k, float sm_scale,
                                         float* out_partial, float* lse_partial, void* stream) {
  g_err.clear();
  sma_status s = validate_dcp(rank, dcp_size, q, kv_local, kv_scale_local, kv_dtype, n_k_local, idx, n_q, top_k,
                              sm_scale, out_partial, lse_partial);
  if (s != SMA_OK || n_q == 0) return s;
  const size_t idx_bytes = align_up((size_t)n_q * (size_t)top_k * 4, 256);
  if (idx_bytes > kStaticScratchBytes)
    return fail(SMA_ERR_WORKSPACE,
                "n_q * top_k = %lld index entries (%zu bytes) exceed the %zu-byte static scratch "
                "(at most %zu entries)", (long long)n_q * top_k, idx_bytes, kStaticScratchBytes,
                kStaticScratchBytes / 4);
  if ((s = check_device()) != SMA_OK) return s;
  uint8_t* ws = nullptr;
  if ((s = static_scratch(&ws)) != SMA_OK) return s;
  SMA_DEBUG_RANGE(idx, (int64_t)n_q * top_k, -1, INT32_MAX, "idx", (hipStream_t)stream);
  SMA_DEBUG_POISON(ws, kStaticScratchBytes, (hipStream_t)stream);
  return run_dcp_partial(rank, dcp_size, q, kv_local, kv_scale_local, kv_dtype, n_k_local, idx, n_q, top_k,
                         sm_scale, out_partial, lse_partial, ws, kStaticScratchBytes, (hipStream_t)stream);
}

sma_status sma_lse_merge(const float* parts, const float* lses, int32_t n_part, int32_t n_q, void* out,
                         int32_t out_dtype, float* lse_out, void* stream) {
  g_err.clear();
  SMA_CHECK(n_part >= 1 && n_part <= sma::kMaxMergeParts, "n_part = %d out of [1, %d]", n_part,
            sma::kMaxMergeParts);
  SMA_CHECK(n_q >= 0 && n_q <= (1 << 28), "n_q = %d out of [0, 2^28]", n_q);
  SMA_CHECK(out_dtype == SMA_DT_BF16 || out_dtype == SMA_DT_FP32, "out_dtype = %d", out_dtype);
  if (n_q == 0) return SMA_OK;
  SMA_CHECK(parts && lses && out, "parts, lses and out must be non-NULL");
  SMA_CHECK(aligned(parts, 16), "parts not 16-byte aligned");
  SMA_CHECK(aligned(out, out_dtype == SMA_DT_FP32 ? 16 : 8), "out not aligned");
  sma_status s = check_device();
  if (s != SMA_OK) return s;
  hipError_t e = sma::launch_lse_merge(parts, lses, n_part, n_q, out, out_dtype == SMA_DT_FP32, lse_out,
                                       (hipStream_t)stream);
  return e == hipSuccess ? SMA_OK : hip_fail(e, "lse_merge launch");
}

size_t sma_workspace_bytes(int32_t op, int32_t n_q, int64_t n_k, int32_t top_k, int32_t h_idx,
                           int32_t d_idx) {
  (void)h_idx;
  (void)d_idx;
  if (n_q < 0 || n_k < 1 || top_k < 1) return 0;
  switch (op) {
    case SMA_OP_INDEX_SCORES:
      return 0;
    case SMA_OP_TOPK:   // optional: lets rows longer than 65,536 scores split across workgroups
      return sma::topk_long_wanted(n_k) ? align_up(sma::topk_long_bytes(n_q, n_k, top_k), 256) : 0;
    case SMA_OP_SPARSE_MLA:   // optional: lets small batches split each query's rows
      return align_up(sma::mla_split_bytes(n_q, sma::mla_split_count(n_q, top_k)), 256);
    case SMA_OP_DCP_PARTIAL:   // the rank's local index list, then a small batch's row slices
      return align_up((size_t)n_q * (size_t)top_k * 4, 256) +
             align_up(sma::mla_split_bytes(n_q, sma::mla_split_count(n_q, top_k)), 256);
    case SMA_OP_DENSE_MHA:   // the expanded keys and values, bf16
      return sma::dense_mha_ws_bytes(n_k);
    case SMA_OP_PREFILL:
    case SMA_OP_PCP_SHARE: {
      const int32_t blk = n_q < kMinScoreBlock ? n_q : kMinScoreBlock;
      return prefill_fixed_bytes(n_q, top_k, true, op == SMA_OP_PCP_SHARE) + score_block_bytes(blk, n_k, top_k);
    }
    default:
      return 0;
  }
}

sma_status sma_prefill(const uint16_t* q_idx, const float* w, int64_t w_stride, const void* k_idx,
                       const float* k_scale, int32_t k_dtype, const uint16_t* q, const void* kv,
                       const float* kv_scale, int32_t kv_dtype, const int32_t* q_pos, int32_t n_q,
                       int64_t n_k, int32_t h_idx, int32_t d_idx, int32_t top_k, float sm_scale,
                       void* out, int32_t out_dtype, float* lse, int32_t* idx_out, void* ws,
                       size_t ws_bytes, void* stream) {
  g_err.clear();
  sma_status s = validate_indexer(q_idx, w, w_stride, k_idx, k_scale, k_dtype, q_pos, n_q, n_k, h_idx, d_idx);
  if (s != SMA_OK) return s;
  return prefill_entry(q_idx, nullptr, w, w_stride, k_idx, k_scale, k_dtype, q, kv, kv_scale, kv_dtype, q_pos,
                       n_q, n_k, h_idx, d_idx, top_k, sm_scale, out, out_dtype, lse, idx_out, ws, ws_bytes,
                       stream);
}

sma_status sma_prefill_fp8_indexer(const uint8_t* q_idx, const float* q_scale, const float* w, int64_t w_stride,
                                   const uint8_t* k_idx, const float* k_scale, const uint16_t* q, const void* kv,
                                   const float* kv_scale, int32_t kv_dtype, const int32_t* q_pos, int32_t n_q,
                                   int64_t n_k, int32_t h_idx, int32_t d_idx, int32_t top_k, float sm_scale,
                                   void* out, int32_t out_dtype, float* lse, int32_t* idx_out, void* ws,
                                   size_t ws_bytes, void* stream) {
  g_err.clear();
  sma_status s = validate_indexer_fp8(q_idx, q_scale, w, w_stride, k_idx, k_scale, q_pos, n_q, n_k, h_idx, d_idx);
  if (s != SMA_OK) return s;
  return prefill_entry(q_idx, q_scale, w, w_stride, k_idx, k_scale, SMA_DT_FP8_E4M3, q, kv, kv_scale, kv_dtype,
                       q_pos, n_q, n_k, h_idx, d_idx, top_k, sm_scale, out, out_dtype, lse, idx_out, ws, ws_bytes,
                       stream);
}

sma_status sma_pcp_rank_share(int32_t rank, int32_t pcp_size, int64_t L_total, const uint16_t* q_idx_share,
                              const float* w_share, int64_t w_stride, const void* k_idx,
                              const float* k_scale, int32_t k_dtype, const uint16_t* q_share,
                              const void* kv, const float* kv_scale, int32_t kv_dtype, int32_t h_idx,
                              int32_t d_idx, int32_t top_k, float sm_scale, void* out_share,
                              int32_t out_dtype, float* lse_share, int32_t* idx_share, void* ws,
                              size_t ws_bytes, void* stream) {
  g_err.clear();
  SMA_CHECK(pcp_size >= 1, "pcp_size = %d < 1", pcp_size);
  SMA_CHECK(rank >= 0 && rank < pcp_size, "rank = %d not in [0, %d)", rank, pcp_size);
  const int64_t n_chunks = 2 * (int64_t)pcp_size;   // 64-bit: no overflow for any pcp_size
  SMA_CHECK(L_total >= n_chunks && L_total % n_chunks == 0,
            "L_total = %lld is not a positive multiple of 2*pcp_size = %lld", (long long)L_total,
            (long long)n_chunks);
  SMA_CHECK(L_total <= kMaxKeys, "L_total too large");
  const int64_t n_q64 = L_total / pcp_size;   // two chunks of L_total / (2 pcp_size)
  SMA_CHECK(n_q64 <= 0x7FFFFFFF, "share too large");
  const int32_t n_q = (int32_t)n_q64;
  sma_status s = validate_indexer(q_idx_share, w_share, w_stride, k_idx, k_scale, k_dtype,
                                  nullptr, n_q, L_total, h_idx, d_idx, false);
  if (s != SMA_OK) return s;
  if ((s = validate_mla(q_share, kv, kv_scale, kv_dtype, L_total, idx_share, n_q, top_k, sm_scale,
                        out_share, out_dtype, true)) != SMA_OK)
    return s;
  const size_t fixed = prefill_fixed_bytes(n_q, top_k, idx_share == nullptr, true);
  const int32_t blk = n_q < kMinScoreBlock ? n_q : kMinScoreBlock;
  const size_t need = fixed + score_block_bytes(blk, L_total, top_k);
  if (ws_bytes < need || ws == nullptr)
    return fail(SMA_ERR_WORKSPACE, "workspace %zu bytes < required %zu", ws_bytes, need);
  SMA_CHECK(aligned(ws, 256), "workspace not 256-byte aligned");
  if ((s = check_device()) != SMA_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  SMA_DEBUG_POISON(ws, ws_bytes, st);
  uint8_t* p = static_cast<uint8_t*>(ws);
  int32_t* pos = reinterpret_cast<int32_t*>(p);
  p += align_up((size_t)n_q * 4, 256);
  int32_t* idx = idx_share;
  if (!idx) {
    idx = reinterpret_cast<int32_t*>(p);
    p += align_up((size_t)n_q * top_k * 4, 256);
  }
  hipError_t e = sma::launch_pcp_positions(pos, rank, pcp_size, L_total, st);
  if (e != hipSuccess) return hip_fail(e, "pcp positions launch");
  return run_prefill(q_idx_share, nullptr, w_share, w_stride, k_idx, k_scale, k_dtype, q_share, kv, kv_scale,
                     kv_dtype, pos, n_q, L_total, h_idx, d_idx, top_k, sm_scale, out_share, out_dtype,
                     lse_share, idx, p, ws_bytes - (size_t)(p - static_cast<uint8_t*>(ws)), st);
}

const char* sma_last_error(void) { return g_err.c_str(); }

int32_t sma_version(void) { return (1 << 16) | 0; }

int32_t sma_build_flags(void) { return SMA_DEBUG_CHECKS ? SMA_BUILD_DEBUG_CHECKS : 0; }

}  // extern "C"

namespace sma {

__global__ void pcp_positions_kernel(int32_t* pos, int32_t rank, int32_t nchunk, int32_t c) {
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= 2 * c) return;
  pos[j] = j < c ? rank * c + j : (nchunk - 1 - rank) * c + (j - c);
}

hipError_t launch_pcp_positions(int32_t* pos, int32_t rank, int32_t pcp_size, int64_t L_total,
                                hipStream_t st) {
  const int32_t nchunk = 2 * pcp_size;
  const int32_t c = (int32_t)(L_total / nchunk);
  const int n = 2 * c;
  hipLaunchKernelGGL(pcp_positions_kernel, dim3((n + 255) / 256), dim3(256), 0, st, pos, rank, nchunk, c);
  return hipGetLastError();
}

int device_cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = g_dev_cus[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    g_dev_cus[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

}  // namespace sma
