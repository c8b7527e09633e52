// Indexer score kernel (gfx950).
//
// I[i,s] = sum_h w[i,h] * ReLU(q_I[i,h,:] . k_I[s,:]) for s <= p_i: the
// indexer of the GLM-5.3 part 2 article ("Pourquoi pas TP ou DP ?") that
// scores every earlier token, with the ReLU / head-weight / causal reading.
//
// Shape of the work: a GEMM with M = (query, head) rows, N = keys and
// K = d_I, followed by a per-query reduction over the head rows.  One wave
// keeps its queries' q_I rows resident in registers as MFMA A operands for
// the whole key sweep; the key rows stream through a double-buffered LDS
// tile shared by the workgroup's waves (B operands of
// v_mfma_f32_32x32x16_bf16).  In the 32x32 accumulator a lane holds 16 head
// rows of one key column, so the head reduction is 16 in-lane FMAs plus one
// exchange with the lane 32 apart.
#include "sma_device.h"
#include "sma_launch.h"

namespace sma {

template <int H, int DI>
struct IdxGeom {
  static constexpr int MT = H >= 32 ? H / 32 : 1;   // 32-row M tiles per wave
  static constexpr int QW = 32 * MT / H;            // queries per wave
  static constexpr int KS = DI / 16;                // k-steps per tile
  static constexpr int WAVES = 4;
  static constexpr int QB = QW * WAVES;             // queries per workgroup
  static constexpr int NT = 2;                      // 32-key N tiles per LDS tile
  static constexpr int KT = 32 * NT;                // keys per LDS tile
  static constexpr int ROWB = DI * 2 + 16;          // padded LDS row, bytes
  static constexpr int CHUNKS_BF16 = KT * DI / 8 / 256;   // 16-byte loads per thread
  static constexpr int CHUNKS_FP8 = KT * DI / 16 / 256;
};

template <int H, int DI, bool FP8>
__global__ __launch_bounds__(256, 2) void idx_score_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, int64_t w_stride,
    const void* __restrict__ k_idx, const float* __restrict__ k_scale,
    const int32_t* __restrict__ q_pos, int n_q, int n_k, float* __restrict__ scores, int64_t ld,
    int n_qblocks, int n_chunks, int chunk_keys) {
  using G = IdxGeom<H, DI>;
  constexpr int MT = G::MT, QW = G::QW, KS = G::KS, QB = G::QB, NT = G::NT, KT = G::KT,
                ROWB = G::ROWB;
  __shared__ __attribute__((aligned(16))) uint8_t s_k[2][KT * ROWB];
  __shared__ float s_scale[2][KT];
  __shared__ int s_pos[QB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Later query blocks carry longer causal prefixes: hand them out first.
  const int qb = n_qblocks - 1 - (int)(blockIdx.x / n_chunks);
  const int chunk = (int)(blockIdx.x % n_chunks);
  const int q0 = qb * QB;

  if (tid < QB) {
    const int qi = q0 + tid;
    int p = qi < n_q ? q_pos[qi] : -1;
    s_pos[tid] = p < -1 ? -1 : (p > n_k - 1 ? n_k - 1 : p);
  }
  __syncthreads();
  int pmax = -1;
#pragma unroll
  for (int t = 0; t < QB; ++t) pmax = max(pmax, s_pos[t]);
  const int k_begin = chunk * chunk_keys;
  const int k_end = min(k_begin + chunk_keys, pmax + 1);
  if (k_begin >= k_end) return;   // uniform across the workgroup

  // ---- A operands (q_I rows) and head weights, resident for the sweep ----
  const int lrow = lane & 31, khalf = lane >> 5;
  bf16x8 a[MT][KS];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int row = 32 * t + lrow;
    const int qi = min(q0 + wave * QW + row / H, n_q - 1);
    const uint16_t* src = q_idx + ((int64_t)qi * H + (row % H)) * DI + khalf * 8;
#pragma unroll
    for (int j = 0; j < KS; ++j) a[t][j] = *reinterpret_cast<const bf16x8*>(src + j * 16);
  }
  float wv[MT][16];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const int row = 32 * t + 8 * (jj / 4) + 4 * khalf + (jj % 4);
      const int qi = min(q0 + wave * QW + row / H, n_q - 1);
      wv[t][jj] = w[(int64_t)qi * w_stride + (row % H)];
    }
  int mypos[QW];
#pragma unroll
  for (int q = 0; q < QW; ++q) mypos[q] = s_pos[wave * QW + q];

  // ---- key tile staging: global -> registers -> LDS ----
  constexpr int NCH = FP8 ? G::CHUNKS_FP8 : G::CHUNKS_BF16;
  u32x4 stage[NCH > 0 ? NCH : 1];
  float stage_sc = 0.f;
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int r = 0; r < NCH; ++r) {
      const int c = tid + 256 * r;
      if constexpr (FP8) {
        const int key = c / (DI / 16), col = c % (DI / 16);
        const int gk = min(k0 + key, n_k - 1);
        stage[r] = *reinterpret_cast<const u32x4*>(
            static_cast<const uint8_t*>(k_idx) + (int64_t)gk * DI + col * 16);
      } else {
        const int key = c / (DI / 8), col = c % (DI / 8);
        const int gk = min(k0 + key, n_k - 1);
        stage[r] = *reinterpret_cast<const u32x4*>(
            static_cast<const uint16_t*>(k_idx) + (int64_t)gk * DI + col * 8);
      }
    }
    if constexpr (FP8) {
      if (tid < KT) stage_sc = k_scale[min(k0 + tid, n_k - 1)];
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < NCH; ++r) {
      const int c = tid + 256 * r;
      if constexpr (FP8) {
        const int key = c / (DI / 16), col = c % (DI / 16);
        uint8_t* dst = &s_k[buf][key * ROWB + col * 32];
        u32x4 lo, hi;
        u32x2 t0 = e4m3x4_to_bf16x4(stage[r][0]), t1 = e4m3x4_to_bf16x4(stage[r][1]);
        u32x2 t2 = e4m3x4_to_bf16x4(stage[r][2]), t3 = e4m3x4_to_bf16x4(stage[r][3]);
        lo[0] = t0[0]; lo[1] = t0[1]; lo[2] = t1[0]; lo[3] = t1[1];
        hi[0] = t2[0]; hi[1] = t2[1]; hi[2] = t3[0]; hi[3] = t3[1];
        *reinterpret_cast<u32x4*>(dst) = lo;
        *reinterpret_cast<u32x4*>(dst + 16) = hi;
      } else {
        const int key = c / (DI / 8), col = c % (DI / 8);
        *reinterpret_cast<u32x4*>(&s_k[buf][key * ROWB + col * 16]) = stage[r];
      }
    }
    if constexpr (FP8) {
      if (tid < KT) s_scale[buf][tid] = stage_sc;
    }
  };

  load_tile(k_begin);
  store_tile(0);
  __syncthreads();

  int it = 0;
  for (int k0 = k_begin; k0 < k_end; k0 += KT, ++it) {
    const int buf = it & 1;
    const bool has_next = k0 + KT < k_end;
    if (has_next) load_tile(k0 + KT);

#pragma unroll
    for (int u = 0; u < NT; ++u) {
      f32x16 c[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) c[t] = f32x16{};
      const uint8_t* brow = &s_k[buf][(32 * u + lrow) * ROWB + khalf * 16];
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        const bf16x8 b = *reinterpret_cast<const bf16x8*>(brow + j * 32);
#pragma unroll
        for (int t = 0; t < MT; ++t)
          c[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[t][j], b, c[t], 0, 0, 0);
      }
      // ReLU, head weight, sum over this lane's 16 head rows ...
      float part[QW];
#pragma unroll
      for (int q = 0; q < QW; ++q) part[q] = 0.f;
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          const int ql = (32 * t + 8 * (jj / 4)) / H;
          part[ql] = fmaf(wv[t][jj], fmaxf(c[t][jj], 0.f), part[ql]);
        }
      // ... and the other 16 rows held by the lane 32 apart.
#pragma unroll
      for (int q = 0; q < QW; ++q) part[q] += __shfl_xor(part[q], 32, 64);

      const int key = k0 + 32 * u + lrow;
      float sc = 1.f;
      if constexpr (FP8) sc = s_scale[buf][32 * u + lrow];
#pragma unroll
      for (int q = 0; q < QW; ++q) {
        if ((q & 1) != khalf) continue;   // lanes 0-31 write even queries, 32-63 odd
        const int qi = q0 + wave * QW + q;
        if (qi < n_q && key <= mypos[q]) scores[(int64_t)qi * ld + key] = part[q] * sc;
      }
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }
}

template <int H, int DI, bool FP8>
static hipError_t launch_idx(const IdxArgs& A, hipStream_t st) {
  using G = IdxGeom<H, DI>;
  const int n_qblocks = (A.n_q + G::QB - 1) / G::QB;
  // Split the key range only when there are too few query blocks to fill
  // the chip (decode-shaped batches); prefill keeps one sweep per block.
  int n_chunks = 1;
  const int target_wgs = 2048;
  if (n_qblocks < target_wgs) n_chunks = (target_wgs + n_qblocks - 1) / n_qblocks;
  int chunk_keys = (int)((A.n_k + n_chunks - 1) / n_chunks);
  chunk_keys = ((chunk_keys + G::KT - 1) / G::KT) * G::KT;
  if (chunk_keys < 4 * G::KT) chunk_keys = 4 * G::KT;
  n_chunks = (int)((A.n_k + chunk_keys - 1) / chunk_keys);
  const long long grid = (long long)n_qblocks * n_chunks;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((idx_score_kernel<H, DI, FP8>), dim3((unsigned)grid), dim3(256), 0, st,
                     A.q_idx, A.w, A.w_stride, A.k_idx, A.k_scale, A.q_pos, A.n_q, (int)A.n_k,
                     A.scores, A.ld, n_qblocks, n_chunks, chunk_keys);
  return hipGetLastError();
}

hipError_t launch_index_scores(const IdxArgs& A, hipStream_t st) {
  const bool f8 = A.fp8;
#define SMA_IDX_CASE(HH, DD)                                                          \
  if (A.h_idx == HH && A.d_idx == DD)                                                 \
    return f8 ? launch_idx<HH, DD, true>(A, st) : launch_idx<HH, DD, false>(A, st);
  SMA_IDX_CASE(64, 128)
  SMA_IDX_CASE(64, 64)
  SMA_IDX_CASE(32, 128)
  SMA_IDX_CASE(32, 64)
  SMA_IDX_CASE(16, 128)
  SMA_IDX_CASE(16, 64)
  SMA_IDX_CASE(8, 128)
  SMA_IDX_CASE(8, 64)
#undef SMA_IDX_CASE
  return hipErrorInvalidValue;
}

}  // namespace sma
