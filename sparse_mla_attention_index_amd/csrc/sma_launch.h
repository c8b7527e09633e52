// Internal launch interface between the C ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#define SMA_MAX_TOPK_DEV 2048

namespace sma {

// Compute units of the current device (queried once per device, kept in an
// atomic per-device cache; 256 if the query fails).
int device_cu_count();

struct IdxArgs {
  const void* q_idx;        // bf16 rows, or e4m3fn codes when q_scale is set
  const float* q_scale = nullptr;   // FP8 queries: one scale per (query, head) row
  const float* w;
  int64_t w_stride;
  const void* k_idx;
  const float* k_scale;
  bool fp8;
  const int32_t* q_pos;
  int32_t n_q;
  int64_t n_k;
  int32_t h_idx, d_idx;
  float* scores;
  int64_t ld;
};

struct TopkArgs {
  const float* scores;
  int64_t ld;
  const int32_t* q_pos;
  int32_t n_q;
  int64_t n_k;
  int32_t top_k;
  int32_t* idx;
  // Workspace for rows split across workgroups (may be null: then long rows
  // take the single-workgroup streaming kernel).
  void* ws = nullptr;
  size_t ws_bytes = 0;
};

struct MlaArgs {
  const uint16_t* q;
  const void* kv;
  const float* kv_scale;
  bool fp8;
  int64_t n_k;
  const int32_t* idx;
  int32_t n_q, top_k;
  float sm_scale;
  void* out;
  bool out_f32;
  float* lse;
  // Workspace for the split partials of small batches (may be null).
  void* ws = nullptr;
  size_t ws_bytes = 0;
  // fp8 && ds_mla: 656-byte fp8_ds_mla rows (scales inside the row, kv_scale unused)
  bool ds_mla = false;
};

// Number of row slices per query the attention kernel uses for n_q
// queries (1: no split), and the workspace bytes their partials take.
int mla_split_count(int n_q, int top_k);
size_t mla_split_bytes(int n_q, int n_split);

hipError_t launch_index_scores(const IdxArgs& a, hipStream_t s);
// e4m3fn rows of d = 64 or 128 values -> codes + one fp32 scale per row.
hipError_t launch_quantize_fp8_rows(const uint16_t* x, int64_t n_rows, int d, uint8_t* codes, float* scale,
                                    hipStream_t s);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
// Rows longer than 65,536 scores, when too few to fill the device one per
// workgroup, are split across workgroups if the workspace holds
// topk_long_bytes(n_q, n_k, top_k).
bool topk_long_wanted(int64_t n_k);
size_t topk_long_bytes(int32_t n_q, int64_t n_k, int32_t top_k);
hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t s);

// DCP share: the tokens of a query's selection that rank `rank` of P stores
// (s mod P == rank), as local rows s / P, ascending, -1 padded.
hipError_t launch_dcp_local_idx(const int32_t* idx, int n_q, int K, int rank, int P, int64_t n_k_local,
                                int32_t* local, hipStream_t s);
// Log-sum-exp merge of n_part partial results [n_part, n_q, 64, 512] fp32
// with their lse [n_part, n_q, 64].
constexpr int kMaxMergeParts = 64;
hipError_t launch_lse_merge(const float* parts, const float* lses, int n_part, int n_q, void* out, bool out_f32,
                            float* lse_out, hipStream_t s);
// Batched bf16 product C_h = A_h . B_h (fp32 accumulation, bf16 out) for
// h < batch: A_h[m][k] at A + h*a_bs + m*lda + k; B_h[k][n] at
// B + h*b_bs + k*ldb + n when b_kn, else at B + h*b_bs + n*ldb + k;
// C_h[m][n] at C + h*c_bs + m*ldc + n.  Requires N % 128 == 0, K % 64 == 0,
// 16-byte aligned rows.
struct BmmArgs {
  const uint16_t* A;
  int64_t lda, a_bs;
  const uint16_t* B;
  int64_t ldb, b_bs;
  bool b_kn;
  uint16_t* C;
  int64_t ldc, c_bs;
  int M, N, K, batch;
};
hipError_t launch_bmm_bf16(const BmmArgs& a, hipStream_t s);

// Dense causal MHA prefill over the latent expanded per head: q [n_q, 64,
// 192] (128 no-rope + 64 rope), kv [n_k, 576] latent rows, w_uk / w_uv [64,
// 128, 512]; ws holds the expanded keys and values (dense_mha_ws_bytes).
struct DenseMhaArgs {
  const uint16_t* q;
  const uint16_t* kv;
  const uint16_t* w_uk;
  const uint16_t* w_uv;
  const int32_t* q_pos;
  int32_t n_q;
  int64_t n_k;
  float sm_scale;
  void* out;
  bool out_f32;
  float* lse;
  void* ws;
};
size_t dense_mha_ws_bytes(int64_t n_k);
hipError_t launch_dense_mha(const DenseMhaArgs& a, hipStream_t s);

hipError_t launch_pcp_positions(int32_t* pos, int32_t rank, int32_t pcp_size, int64_t L_total,
                                hipStream_t s);

}  // namespace sma
