// Host-side driver for the sanitizer build of the C ABI layer (ASan + UBSan
// on the host code of csrc/sma_api.hip).  Every entry point is called with
// arguments its validation rejects, and the workspace-size arithmetic is
// run at the largest sizes it accepts; each rejection must come back as the
// documented status with a message, before anything touches a device.  With
// no device present, calls that pass validation stop at the device check.
// Prints "abi_driver ok" and exits 0 when every expectation holds; the
// sanitizers abort the process on any memory error or undefined behaviour.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <limits>

#include "sma.h"

static int g_fail = 0;

static void expect(sma_status got, sma_status want, const char* needle, const char* what) {
  const char* msg = sma_last_error();
  if (got != want || (needle && !std::strstr(msg, needle))) {
    std::printf("FAIL %s: status %d (want %d), message \"%s\"\n", what, (int)got, (int)want, msg);
    ++g_fail;
  }
}

int main() {
  // any non-null pointer: never dereferenced on the host, and no call below
  // reaches a kernel launch
  static uint8_t fake_storage[4096] __attribute__((aligned(256)));
  void* F = fake_storage;
  const uint16_t* F16 = reinterpret_cast<const uint16_t*>(F);
  const float* Ff = reinterpret_cast<const float*>(F);
  const int32_t* Fi = reinterpret_cast<const int32_t*>(F);
  const uint8_t* F8 = reinterpret_cast<const uint8_t*>(F);
  const float nan = std::numeric_limits<float>::quiet_NaN();

  // indexer
  expect(sma_index_scores(F16, Ff, 64, F, nullptr, 0, Fi, 1, 10, 7, 128, (float*)F, 10, nullptr), SMA_ERR_UNSUPPORTED,
         "h_idx", "index_scores h_idx");
  expect(sma_index_scores(F16, Ff, 64, nullptr, nullptr, 0, Fi, 1, 10, 64, 128, (float*)F, 10, nullptr),
         SMA_ERR_INVALID_ARG, "k_idx", "index_scores null keys");
  expect(sma_index_scores(F16, Ff, 64, F, nullptr, 0, Fi, 1, 10, 64, 128, (float*)F, 9, nullptr), SMA_ERR_INVALID_ARG,
         "ld_scores", "index_scores ld");
  expect(sma_index_scores(F16, Ff, 64, F, nullptr, 0, Fi, -1, 10, 64, 128, (float*)F, 10, nullptr),
         SMA_ERR_INVALID_ARG, "n_q", "index_scores n_q");
  expect(sma_index_scores(F16, Ff, 64, F, nullptr, 0, Fi, 1, (int64_t)1 << 40, 64, 128, (float*)F, (int64_t)1 << 40,
                          nullptr), SMA_ERR_INVALID_ARG, "n_k", "index_scores huge n_k");
  expect(sma_index_scores(F16, Ff, 64, F, nullptr, 0, Fi, 0, 10, 64, 128, (float*)F, 10, nullptr), SMA_OK, nullptr,
         "index_scores n_q = 0 no-op");
  expect(sma_index_scores_fp8(F8, Ff, Ff, 64, F8, Ff, Fi, 1, 10, 32, 128, (float*)F, 10, nullptr), SMA_ERR_UNSUPPORTED,
         "64 x 128", "index_scores_fp8 shape");
  expect(sma_quantize_fp8_rows(F16, (int64_t)1 << 40, 128, (uint8_t*)F, (float*)F, nullptr), SMA_ERR_INVALID_ARG,
         "n_rows", "quantize n_rows");
  // top-k
  expect(sma_topk_select(Ff, 10, Fi, 1, 10, 0, (int32_t*)F, nullptr, 0, nullptr), SMA_ERR_INVALID_ARG, "top_k",
         "topk top_k 0");
  expect(sma_topk_select(Ff, 10, Fi, 1, 10, 2049, (int32_t*)F, nullptr, 0, nullptr), SMA_ERR_INVALID_ARG, "top_k",
         "topk top_k 2049");
  expect(sma_topk_select(Ff, 10, Fi, 1, 10, 8, (int32_t*)F, (uint8_t*)F + 4, 64, nullptr), SMA_ERR_INVALID_ARG,
         "aligned", "topk misaligned workspace");
  // sparse MLA
  for (float sc : {0.f, -1.f, nan, std::numeric_limits<float>::infinity()})
    expect(sma_sparse_mla_prefill(F16, F, nullptr, 0, 100, Fi, 1, 8, sc, F, 0, nullptr, nullptr, 0, nullptr),
           SMA_ERR_INVALID_ARG, "sm_scale", "mla sm_scale");
  expect(sma_sparse_mla_prefill(F16, F, Ff, 0, 100, Fi, 1, 8, 0.1f, F, 0, nullptr, nullptr, 0, nullptr),
         SMA_ERR_INVALID_ARG, "kv_scale", "mla bf16 with scale");
  expect(sma_sparse_mla_prefill(F16, F, nullptr, 9, 100, Fi, 1, 8, 0.1f, F, 0, nullptr, nullptr, 0, nullptr),
         SMA_ERR_INVALID_ARG, "kv_dtype", "mla kv_dtype");
  // composed paths
  expect(sma_prefill(F16, Ff, 64, F, nullptr, 0, F16, F, nullptr, 0, Fi, 16, 1000, 64, 128, 64, 0.1f, F, 0, nullptr,
                     nullptr, F, 100, nullptr), SMA_ERR_WORKSPACE, "workspace", "prefill small workspace");
  expect(sma_prefill_fp8_indexer(F8, Ff, Ff, 64, F8, Ff, F16, F, nullptr, 0, Fi, 16, 1000, 64, 128, 64, 0.1f, F, 0,
                                 nullptr, nullptr, F, 100, nullptr), SMA_ERR_WORKSPACE, "workspace",
         "prefill_fp8 small workspace");
  expect(sma_pcp_rank_share(8, 8, 1024, F16, Ff, 64, F, nullptr, 0, F16, F, nullptr, 0, 64, 128, 2048, 0.1f, F, 0,
                            nullptr, nullptr, F, (size_t)1 << 40, nullptr), SMA_ERR_INVALID_ARG, "rank", "pcp rank");
  expect(sma_pcp_rank_share(0, 8, 1000, F16, Ff, 64, F, nullptr, 0, F16, F, nullptr, 0, 64, 128, 2048, 0.1f, F, 0,
                            nullptr, nullptr, F, (size_t)1 << 40, nullptr), SMA_ERR_INVALID_ARG, "L_total",
         "pcp L_total");
  expect(sma_pcp_rank_share(0, INT32_MAX, 1024, F16, Ff, 64, F, nullptr, 0, F16, F, nullptr, 0, 64, 128, 2048, 0.1f,
                            F, 0, nullptr, nullptr, F, (size_t)1 << 40, nullptr), SMA_ERR_INVALID_ARG, nullptr,
         "pcp huge pcp_size");
  // absorption, dense MHA, DCP, merge
  expect(sma_absorb_q(F16, F16, 4, 64, (uint16_t*)F, 500, nullptr), SMA_ERR_INVALID_ARG, "ld_out", "absorb ld_out");
  expect(sma_project_out(F16, F16, 4, 2000, (uint16_t*)F, nullptr), SMA_ERR_INVALID_ARG, "heads", "project heads");
  expect(sma_dense_mha_prefill(F16, F16, F16, F16, Fi, 4, 100, 0.1f, F, 0, nullptr, F, 100 * 32768 - 1, nullptr),
         SMA_ERR_WORKSPACE, "workspace", "dense mha workspace");
  expect(sma_dense_mha_prefill(F16, F16, F16, F16, Fi, 4, 100, -0.1f, F, 0, nullptr, F, 1 << 30, nullptr),
         SMA_ERR_INVALID_ARG, "sm_scale", "dense mha scale");
  expect(sma_dcp_shard_partial(3, 3, F16, F, nullptr, 0, 100, Fi, 1, 8, 0.1f, (float*)F, (float*)F, F, 1 << 20,
                               nullptr), SMA_ERR_INVALID_ARG, "rank", "dcp rank");
  expect(sma_dcp_shard_partial_noalloc(0, 2, F16, F, nullptr, 0, 100, Fi, 8193, 2048, 0.1f, (float*)F, (float*)F,
                                       nullptr), SMA_ERR_WORKSPACE, "static scratch", "dcp noalloc limit");
  expect(sma_lse_merge(Ff, Ff, 65, 3, F, 0, nullptr, nullptr), SMA_ERR_INVALID_ARG, "n_part", "merge n_part");
  // a call that passes validation stops at the device check (no device here)
  const sma_status dev = sma_lse_merge(Ff, Ff, 2, 3, F, 0, nullptr, nullptr);
  if (dev == SMA_OK || std::strlen(sma_last_error()) == 0) {
    std::printf("FAIL: a valid call reported %d with message \"%s\" and no device\n", (int)dev, sma_last_error());
    ++g_fail;
  }

  // workspace arithmetic at the extremes: no overflow, no undefined behaviour
  const int32_t nqs[] = {0, 1, 63, 64, 65, 1 << 20, INT32_MAX};
  const int64_t nks[] = {1, 65536, 65537, 1 << 20, ((int64_t)1 << 31) - 1};
  const int32_t tks[] = {1, 2048};
  size_t sink = 0;
  for (int op = -1; op <= 7; ++op)
    for (int32_t nq : nqs)
      for (int64_t nk : nks)
        for (int32_t tk : tks) sink += sma_workspace_bytes(op, nq, nk, tk, 64, 128);
  sink += sma_workspace_bytes(SMA_OP_PREFILL, -5, 10, 8, 64, 128) + sma_workspace_bytes(SMA_OP_TOPK, 5, 0, 8, 64, 128);
  std::printf("workspace checksum %zu\n", sink);

  if ((sma_version() >> 16) != 1) {
    std::printf("FAIL: version %d\n", (int)sma_version());
    ++g_fail;
  }
  if (g_fail) {
    std::printf("abi_driver: %d failures\n", g_fail);
    return 1;
  }
  std::printf("abi_driver ok\n");
  return 0;
}
