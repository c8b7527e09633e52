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
        // codes widened by the hardware convert (exact in fp32 and in bf16)
        uint8_t* dst = &s_k[buf][key * ROWB + col * 32];
        uint32_t packed[8];
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)stage[r][wd], false);
          const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)stage[r][wd], true);
          packed[2 * wd] = pack_bf16x2(lo[0], lo[1]);
          packed[2 * wd + 1] = pack_bf16x2(hi[0], hi[1]);
        }
        *reinterpret_cast<u32x4*>(dst) = u32x4{packed[0], packed[1], packed[2], packed[3]};
        *reinterpret_cast<u32x4*>(dst + 16) = u32x4{packed[4], packed[5], packed[6], packed[7]};
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
                     static_cast<const uint16_t*>(A.q_idx), A.w, A.w_stride, A.k_idx, A.k_scale, A.q_pos, A.n_q,
                     (int)A.n_k,
                     A.scores, A.ld, n_qblocks, n_chunks, chunk_keys);
  return hipGetLastError();
}

// The queries of the workgroup whose block starts at q0 (one per wave, W
// waves): for a batch of at most 64 W queries, those of ranks q0 .. q0 + W -
// 1 in position order (ties by index), so that a block's causal extent, its
// largest position, wastes little on the block's other queries (a decode
// batch's positions come in any order); for larger batches, queries q0 ..
// q0 + W - 1.  Fills s_qid (-1: no query) and s_pos (clamped to [-1, n_k -
// 1]) for the W slots, using s_allpos (64 W ints) as scratch, and ends with
// a barrier.
template <int W>
__device__ __forceinline__ void idx_block_queries(const int32_t* __restrict__ q_pos, int n_q, int n_k, int q0,
                                                  int* s_qid, int* s_pos, int* s_allpos) {
  const int tid = threadIdx.x;
  auto clamp_pos = [&](int p) { return p < -1 ? -1 : (p > n_k - 1 ? n_k - 1 : p); };
  if (n_q <= 64 * W) {
    int p = -1;
    if (tid < n_q) s_allpos[tid] = p = clamp_pos(q_pos[tid]);
    if (tid < W) {
      s_qid[tid] = -1;
      s_pos[tid] = -1;
    }
    __syncthreads();
    if (tid < n_q) {
      int rank = 0;
      for (int j = 0; j < n_q; ++j) {
        const int pj = s_allpos[j];
        rank += (pj < p) || (pj == p && j < tid);
      }
      if (rank >= q0 && rank < q0 + W) {
        s_qid[rank - q0] = tid;
        s_pos[rank - q0] = p;
      }
    }
  } else if (tid < W) {
    const int qi = q0 + tid;
    s_qid[tid] = qi < n_q ? qi : -1;
    s_pos[tid] = qi < n_q ? clamp_pos(q_pos[qi]) : -1;
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// bf16 keys, 64 heads x d_I = 128 (the prefill shape): eight waves, one query
// each, share a ring of key tiles filled by direct global->LDS loads, so a
// key tile read from L2 serves eight queries and up to kIdxStages - 1 tiles
// are in flight while one is consumed.  Two waves per SIMD let one wave's
// ReLU / head-weight epilogue overlap the other's MFMAs.
//
// Tile: 64 keys x 256 bytes, dense; 16-byte chunk c of key r sits at slot
// c ^ (r & 15) of the key's row, so the 16 lanes of a B-operand read (16
// keys, one chunk) hit 16 distinct bank groups.  A 1-KiB load covers four
// keys; lane l fetches key 4b + (l >> 4), slot l & 15.
// ---------------------------------------------------------------------------
constexpr int kIdxWaves = 8;
constexpr int kIdxKT = 64;                                  // keys per tile
constexpr int kIdxStages = 8;                               // ring depth
constexpr int kIdxTileB = kIdxKT * 256;                     // 16 KiB
constexpr int kIdxLoadsPerWave = kIdxTileB / 1024 / kIdxWaves;   // 2

typedef __attribute__((address_space(3))) uint8_t idx_lds_u8;

__device__ __forceinline__ void idx_dma16(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr), "s"(lds_base)
               : "memory", "m0");
}
template <int N>
__device__ __forceinline__ void idx_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void idx_dma4(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gaddr), "s"(lds_base)
               : "memory", "m0");
}

__device__ __forceinline__ void idx_sync_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt not waited
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(64 * kIdxWaves, 1) void idx_score_h64_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, int64_t w_stride,
    const uint16_t* __restrict__ k_idx, const int32_t* __restrict__ q_pos, int n_q, int n_k,
    float* __restrict__ scores, int64_t ld, int n_qblocks, int n_chunks, int chunk_keys) {
  constexpr int H = 64, DI = 128, KS = DI / 16;
  __shared__ __attribute__((aligned(1024))) uint8_t s_k[kIdxStages][kIdxTileB];
  __shared__ int s_pos[kIdxWaves], s_qid[kIdxWaves], s_allpos[64 * kIdxWaves];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Later query blocks carry longer causal prefixes: hand them out first.
  const int qb = n_qblocks - 1 - (int)(blockIdx.x / n_chunks);
  const int chunk = (int)(blockIdx.x % n_chunks);
  const int q0 = qb * kIdxWaves;
  idx_block_queries<kIdxWaves>(q_pos, n_q, n_k, q0, s_qid, s_pos, s_allpos);
  int pmax = -1;
#pragma unroll
  for (int t = 0; t < kIdxWaves; ++t) pmax = max(pmax, s_pos[t]);
  const int k_begin = chunk * chunk_keys;
  const int k_end = min(k_begin + chunk_keys, pmax + 1);
  if (k_begin >= k_end) return;   // uniform across the workgroup
  const int ntiles = (k_end - k_begin + kIdxKT - 1) / kIdxKT;
  const int mypos = s_pos[wave];
  const int myq = s_qid[wave];          // -1: no query in this slot
  const int qi = myq < 0 ? 0 : myq;

  // ---- A operands: the wave's query, head rows 32t + lrow, dims 16j + 8khalf .. +7 ----
  const int lrow = lane & 31, khalf = lane >> 5;
  bf16x8 a[2][KS];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint16_t* src = q_idx + ((int64_t)qi * H + 32 * t + lrow) * DI + khalf * 8;
#pragma unroll
    for (int j = 0; j < KS; ++j) a[t][j] = *reinterpret_cast<const bf16x8*>(src + j * 16);
  }
  // head weights of this lane's accumulator rows 32t + 8(jj>>2) + 4khalf + (jj&3)
  float wv[2][16];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) wv[t][jj] = w[(int64_t)qi * w_stride + 32 * t + 8 * (jj >> 2) + 4 * khalf + (jj & 3)];

  // ---- gather of tile i (keys k_begin + 64i ..) into slot i % kIdxStages ----
  const int dkey = kIdxLoadsPerWave * 4 * wave + (lane >> 4);   // key of load 0 within the tile
  auto issue = [&](int i) {
    const uint32_t dst = (uint32_t)(uintptr_t)(idx_lds_u8*)&s_k[i % kIdxStages][1024 * kIdxLoadsPerWave * wave];
#pragma unroll
    for (int j = 0; j < kIdxLoadsPerWave; ++j) {
      const int key = min(k_begin + kIdxKT * i + dkey + 4 * j, n_k - 1);
      const int c = (lane & 15) ^ ((dkey + 4 * j) & 15);
      idx_dma16(k_idx + (int64_t)key * DI + 8 * c, dst + 1024 * j);
    }
  };
  // Retire the operand loads so that only gathers are outstanding below.
  idx_wait_vmcnt<0>();
#pragma unroll
  for (int i = 0; i < kIdxStages - 1; ++i) issue(i);

  // B operand of N-tile u, k-step j: key 32u + lrow, chunk 2j + khalf at slot (2j + khalf) ^ (lrow & 15).
  int boff[KS];
#pragma unroll
  for (int j = 0; j < KS; ++j) boff[j] = lrow * 256 + 16 * ((2 * j + khalf) ^ (lrow & 15));

  // Software pipeline over 32-key N-tiles: the MFMAs of N-tile n run while
  // the ReLU / head-weight epilogue of N-tile n-1 is issued, so the VALU work
  // hides under the matrix core instead of following it.
  f32x16 acc[2][2] = {{f32x16{}, f32x16{}}, {f32x16{}, f32x16{}}};   // [buffer][M tile]
  int prev_key = -1;  // first key of the N-tile whose sums wait in the other buffer
  auto epilogue = [&](const f32x16& c0, const f32x16& c1, int key0) {
    float part = 0.f;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      // ReLU as an integer max on the float's bits (negative values and -0
      // have the sign bit set): one instruction, no NaN canonicalisation
      part = fmaf(wv[0][jj], __int_as_float(max(__float_as_int(c0[jj]), 0)), part);
      part = fmaf(wv[1][jj], __int_as_float(max(__float_as_int(c1[jj]), 0)), part);
    }
    // lanes 0..31 add the other 32 head rows, held by the lane 32 above
    // (v_permlane32_swap: no LDS round trip inside the MFMA stream)
    part += __uint_as_float(__builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false,
                                                             false)[1]);
    const int key = key0 + lrow;
    if (khalf == 0 && key0 >= 0 && myq >= 0 && key <= mypos && key < k_end)
      scores[(int64_t)myq * ld + key] = part;
  };
  // B operands are read one N-tile ahead of their MFMAs (bn), so the last
  // N-tile of tile i reads tile i + 1: the wait below therefore covers tiles
  // i and i + 1, leaving kIdxStages - 3 tiles in flight.
  idx_wait_vmcnt<(kIdxStages - 2) * kIdxLoadsPerWave>();
  idx_sync_lds();
  bf16x8 bn[KS];
#pragma unroll
  for (int j = 0; j < KS; ++j) bn[j] = *reinterpret_cast<const bf16x8*>(s_k[0] + boff[j]);
  for (int i = 0; i < ntiles; ++i) {
    // tiles i and i + 1 have landed once at most the kIdxStages - 3 younger tiles are outstanding
    idx_wait_vmcnt<(kIdxStages - 3) * kIdxLoadsPerWave>();
    idx_sync_lds();             // for every wave; slot (i - 1) % kIdxStages is free
    issue(i + kIdxStages - 1);  // past the range these load clamped keys into a free slot
    const uint8_t* tile = s_k[i % kIdxStages];
    const int k0 = k_begin + kIdxKT * i;
#pragma unroll
    for (int u = 0; u < kIdxKT / 32; ++u) {
      const f32x16 p0 = acc[(u + 1) & 1][0], p1 = acc[(u + 1) & 1][1];
      // the N-tile after this one: (tile i, u + 1) or (tile i + 1, 0)
      const uint8_t* nxt = u + 1 < kIdxKT / 32 ? tile + 8192 * (u + 1) : s_k[(i + 1) % kIdxStages];
      f32x16 c0 = f32x16{}, c1 = f32x16{};
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        const bf16x8 b = bn[j];
        bn[j] = *reinterpret_cast<const bf16x8*>(nxt + boff[j]);
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][j], b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][j], b, c1, 0, 0, 0);
      }
      epilogue(p0, p1, prev_key);   // the store is skipped before the first N-tile
      acc[u & 1][0] = c0;
      acc[u & 1][1] = c1;
      prev_key = k0 + 32 * u;
      // interleave: one B read (for the next N-tile) and four epilogue VALU
      // instructions per pair of MFMAs
#pragma unroll
      for (int g = 0; g < KS; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x0002, 4, 0);   // VALU
        __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x0002, 4, 0);   // VALU
        __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);   // DS read
      }
    }
  }
  epilogue(acc[(kIdxKT / 32 - 1) & 1][0], acc[(kIdxKT / 32 - 1) & 1][1], prev_key);
  idx_wait_vmcnt<0>();   // no load may land in LDS after the workgroup has left
}

// ---------------------------------------------------------------------------
// bf16 queries over FP8 keys, 64 heads x d_I = 128 (the decode batch): the
// kernel above with an FP8 key ring.  Each wave's direct global->LDS load
// brings 8 keys (1 KiB of codes) and their 8 scales per 64-key tile; once a
// tile has landed, the workgroup widens its codes to bf16 (the hardware
// convert, exact) into one of two bf16 tiles laid out and swizzled as above,
// so the MFMA loop is unchanged; the key's scale multiplies the head sum.
// The convert is v_cvt_scalef32_pk_bf16_fp8 at scale 1 (exact), and the
// barrier that orders a tile's widening before its B-operand reads sits
// between the previous tile's two N-tiles, so the widening overlaps the
// first N-tile's MFMAs instead of stalling every wave before them.
// ---------------------------------------------------------------------------
constexpr int kF8kTileB = kIdxKT * 128;   // 8 KiB of codes per 64-key tile

__global__ __launch_bounds__(64 * kIdxWaves, 1) void idx_score_h64_f8k_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w, int64_t w_stride,
    const uint8_t* __restrict__ k8, const float* __restrict__ k_scale, const int32_t* __restrict__ q_pos, int n_q,
    int n_k, float* __restrict__ scores, int64_t ld, int n_qblocks, int n_chunks, int chunk_keys) {
  constexpr int H = 64, DI = 128, KS = DI / 16;
  __shared__ __attribute__((aligned(1024))) uint8_t s_c8[kIdxStages][kF8kTileB];   // codes, as stored
  __shared__ __attribute__((aligned(16))) float s_sc[kIdxStages][kIdxKT];
  __shared__ __attribute__((aligned(1024))) uint8_t s_k[2][kIdxTileB];             // widened, swizzled
  __shared__ int s_pos[kIdxWaves], s_qid[kIdxWaves], s_allpos[64 * kIdxWaves];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qb = n_qblocks - 1 - (int)(blockIdx.x / n_chunks);
  const int chunk = (int)(blockIdx.x % n_chunks);
  const int q0 = qb * kIdxWaves;
  idx_block_queries<kIdxWaves>(q_pos, n_q, n_k, q0, s_qid, s_pos, s_allpos);
  int pmax = -1;
#pragma unroll
  for (int t = 0; t < kIdxWaves; ++t) pmax = max(pmax, s_pos[t]);
  const int k_begin = chunk * chunk_keys;
  const int k_end = min(k_begin + chunk_keys, pmax + 1);
  if (k_begin >= k_end) return;   // uniform across the workgroup
  const int ntiles = (k_end - k_begin + kIdxKT - 1) / kIdxKT;
  const int mypos = s_pos[wave];
  const int myq = s_qid[wave];          // -1: no query in this slot
  const int qi = myq < 0 ? 0 : myq;

  const int lrow = lane & 31, khalf = lane >> 5;
  bf16x8 a[2][KS];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const uint16_t* src = q_idx + ((int64_t)qi * H + 32 * t + lrow) * DI + khalf * 8;
#pragma unroll
    for (int j = 0; j < KS; ++j) a[t][j] = *reinterpret_cast<const bf16x8*>(src + j * 16);
  }
  float wv[2][16];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) wv[t][jj] = w[(int64_t)qi * w_stride + 32 * t + 8 * (jj >> 2) + 4 * khalf + (jj & 3)];

  // ---- tile i (keys k_begin + 64i ..): codes and scales into ring slot i % kIdxStages ----
  auto issue = [&](int i) {
    const int slot = i % kIdxStages;
    const int kt = k_begin + kIdxKT * i;
    const uint32_t dst = (uint32_t)(uintptr_t)(idx_lds_u8*)&s_c8[slot][1024 * wave];
    idx_dma16(k8 + (int64_t)min(kt + 8 * wave + (lane >> 3), n_k - 1) * DI + 16 * (lane & 7), dst);
    const uint32_t sdst = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)&s_sc[slot][8 * wave];
    if (lane < 8) idx_dma4(k_scale + min(kt + 8 * wave + lane, n_k - 1), sdst);
  };
  constexpr int kLoads = 2;   // per wave per tile: codes, scales
  // widen tile i: thread t takes 16 codes (key t >> 3, 16-byte chunk t & 7)
  // into bf16 chunks 2c and 2c + 1 of the key at slots (2c + h) ^ (key & 15)
  auto widen = [&](int i) {
    const int key = tid >> 3, c = tid & 7;
    const u32x4 v = *reinterpret_cast<const u32x4*>(&s_c8[i % kIdxStages][key * 128 + 16 * c]);
    uint32_t packed[8];
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      packed[2 * wd] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[wd], 1.f, false));
      packed[2 * wd + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[wd], 1.f, true));
    }
    uint8_t* row = &s_k[i & 1][key * 256];
    *reinterpret_cast<u32x4*>(row + 16 * ((2 * c) ^ (key & 15))) = u32x4{packed[0], packed[1], packed[2], packed[3]};
    *reinterpret_cast<u32x4*>(row + 16 * ((2 * c + 1) ^ (key & 15))) =
        u32x4{packed[4], packed[5], packed[6], packed[7]};
  };
  idx_wait_vmcnt<0>();
#pragma unroll
  for (int i = 0; i < kIdxStages - 1; ++i) issue(i);
  int boff[KS];
#pragma unroll
  for (int j = 0; j < KS; ++j) boff[j] = lrow * 256 + 16 * ((2 * j + khalf) ^ (lrow & 15));

  f32x16 acc[2][2] = {{f32x16{}, f32x16{}}, {f32x16{}, f32x16{}}};
  int prev_key = -1;
  float prev_sc = 0.f;
  auto epilogue = [&](const f32x16& c0, const f32x16& c1, int key0, float sc) {
    float part = 0.f;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      part = fmaf(wv[0][jj], __int_as_float(max(__float_as_int(c0[jj]), 0)), part);
      part = fmaf(wv[1][jj], __int_as_float(max(__float_as_int(c1[jj]), 0)), part);
    }
    part += __uint_as_float(__builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false,
                                                             false)[1]);
    const int key = key0 + lrow;
    if (khalf == 0 && key0 >= 0 && myq >= 0 && key <= mypos && key < k_end)
      scores[(int64_t)myq * ld + key] = part * sc;
  };
  // tile 0 widened before the loop; iteration i widens tile i + 1 (whose B
  // operands the last N-tile of tile i reads), so the waits cover tiles i
  // and i + 1, leaving kIdxStages - 3 tiles in flight
  idx_wait_vmcnt<(kIdxStages - 2) * kLoads>();
  idx_sync_lds();
  widen(0);
  idx_sync_lds();
  bf16x8 bn[KS];
#pragma unroll
  for (int j = 0; j < KS; ++j) bn[j] = *reinterpret_cast<const bf16x8*>(s_k[0] + boff[j]);
  float scn = s_sc[0][lrow];
  for (int i = 0; i < ntiles; ++i) {
    idx_wait_vmcnt<(kIdxStages - 3) * kLoads>();
    idx_sync_lds();             // tile i + 1 landed; bf16 tile (i + 1) & 1 is no longer read
    widen(i + 1);               // past the range this widens clamped keys, never stored
    issue(i + kIdxStages - 1);  // into slot (i - 1) % kIdxStages, whose codes were widened at i - 2
    const uint8_t* tile = s_k[i & 1];
    const int slot = i % kIdxStages;
    const int k0 = k_begin + kIdxKT * i;
#pragma unroll
    for (int u = 0; u < kIdxKT / 32; ++u) {
      const f32x16 p0 = acc[(u + 1) & 1][0], p1 = acc[(u + 1) & 1][1];
      const bool last = u + 1 == kIdxKT / 32;
      const uint8_t* nxt = last ? s_k[(i + 1) & 1] : tile + 8192 * (u + 1);
      const float* nsc = last ? &s_sc[(i + 1) % kIdxStages][0] : &s_sc[slot][32 * (u + 1)];
      const float sc = scn;
      f32x16 c0 = f32x16{}, c1 = f32x16{};
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        const bf16x8 b = bn[j];
        bn[j] = *reinterpret_cast<const bf16x8*>(nxt + boff[j]);
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0][j], b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1][j], b, c1, 0, 0, 0);
      }
      scn = nsc[lrow];
      epilogue(p0, p1, prev_key, prev_sc);
      acc[u & 1][0] = c0;
      acc[u & 1][1] = c1;
      prev_key = k0 + 32 * u;
      prev_sc = sc;
#pragma unroll
      for (int g = 0; g < KS; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x0002, 4, 0);   // VALU
        __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x0002, 4, 0);   // VALU
        __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);   // DS read
      }
      if (u == 0) idx_sync_lds();   // tile i + 1 widened before the last N-tile reads it
    }
  }
  epilogue(acc[(kIdxKT / 32 - 1) & 1][0], acc[(kIdxKT / 32 - 1) & 1][1], prev_key, prev_sc);
  idx_wait_vmcnt<0>();
}

static hipError_t launch_idx_h64_f8k(const IdxArgs& A, hipStream_t st) {
  const int n_qblocks = (A.n_q + kIdxWaves - 1) / kIdxWaves;
  int n_chunks = 1;
  const int target_wgs = 1024;
  if (n_qblocks < target_wgs) n_chunks = (target_wgs + n_qblocks - 1) / n_qblocks;
  int chunk_keys = (int)((A.n_k + n_chunks - 1) / n_chunks);
  chunk_keys = ((chunk_keys + kIdxKT - 1) / kIdxKT) * kIdxKT;
  if (chunk_keys < 4 * kIdxKT) chunk_keys = 4 * kIdxKT;
  n_chunks = (int)((A.n_k + chunk_keys - 1) / chunk_keys);
  const long long grid = (long long)n_qblocks * n_chunks;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(idx_score_h64_f8k_kernel, dim3((unsigned)grid), dim3(64 * kIdxWaves), 0, st,
                     static_cast<const uint16_t*>(A.q_idx), A.w, A.w_stride, static_cast<const uint8_t*>(A.k_idx),
                     A.k_scale, A.q_pos, A.n_q, (int)A.n_k, A.scores, A.ld, n_qblocks, n_chunks, chunk_keys);
  return hipGetLastError();
}

static hipError_t launch_idx_h64(const IdxArgs& A, hipStream_t st) {
  const int n_qblocks = (A.n_q + kIdxWaves - 1) / kIdxWaves;
  int n_chunks = 1;
  const int target_wgs = 1024;
  if (n_qblocks < target_wgs) n_chunks = (target_wgs + n_qblocks - 1) / n_qblocks;
  int chunk_keys = (int)((A.n_k + n_chunks - 1) / n_chunks);
  chunk_keys = ((chunk_keys + kIdxKT - 1) / kIdxKT) * kIdxKT;
  if (chunk_keys < 4 * kIdxKT) chunk_keys = 4 * kIdxKT;
  n_chunks = (int)((A.n_k + chunk_keys - 1) / chunk_keys);
  const long long grid = (long long)n_qblocks * n_chunks;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(idx_score_h64_kernel, dim3((unsigned)grid), dim3(64 * kIdxWaves), 0, st,
                     static_cast<const uint16_t*>(A.q_idx), A.w,
                     A.w_stride, static_cast<const uint16_t*>(A.k_idx), A.q_pos, A.n_q, (int)A.n_k, A.scores, A.ld,
                     n_qblocks, n_chunks, chunk_keys);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// FP8 queries and FP8 keys, 64 heads x d_I = 128, on
// v_mfma_scale_f32_32x32x64_f8f6f4, whose e4m3 x e4m3 products run at twice
// the bf16 rate.  Its block scales are left at 2^0: the per-row fp32 scales
// act outside the dot product,
//   w_h * ReLU(sq_h * sk_s * d) = sk_s * (w_h * sq_h) * ReLU(d),  sq, sk >= 0,
// so the head weight absorbs the query row's scale and the key's scale
// multiplies the head sum once.
//
// At twice the MFMA rate the epilogue (a ReLU and an FMA per head and key,
// fp32) issues more VALU cycles than the MFMAs take, so the kernel is laid
// out to keep the VALU busy: twelve waves (three per SIMD), one query each,
// share a ring of 96-key tiles filled by direct global->LDS loads; inside a
// wave the epilogue of one 32-key N-tile is interleaved with the MFMAs of
// the next; stores take their row base and lane mask in scalar registers.
//
// Tile: 96 keys x 128 bytes (12 KiB) plus the 96 key scales.  16-byte chunk
// c of key r sits at slot c ^ ((r >> 1) & 7) of its 128-byte row.  The LDS
// serves 16 lanes of a 16-byte read per cycle over a 256-byte bank period
// (two keys' rows): the 16 lanes that read one chunk of keys r .. r + 15
// then hit 16 distinct 16-byte bank groups (key parity picks the half of
// the period, (r >> 1) & 7 the slot).  Wave v loads keys
// 8v .. 8v + 7 of the tile (one 1-KiB load, lane l taking key 8v + (l >> 3),
// slot l & 7) and their 8 scales (lanes 0..7): every wave issues the same two
// loads per tile and waits on the same counts.
//
// The MFMA's 64-wide K step takes 32 bytes per lane from A and from B.  The
// lane (row, half) loads bytes 64j + 32 half .. +31 of its row for step j in
// both operands; whatever order the instruction assigns those bytes to K
// within the step, it is the same order for A and B, so the step's sum runs
// over exactly the 64 products of matching elements.
// ---------------------------------------------------------------------------
typedef int i32x8 __attribute__((ext_vector_type(8)));
constexpr int kF8Waves = 12;                                 // queries per workgroup
// KL key loads of 1 KiB per wave per tile: KT = 96 KL keys, NT = 3 KL
// N-tiles; a ring of S tiles (a power of two).
template <int KL, int S>
struct F8Geom {
  static constexpr int KT = 8 * kF8Waves * KL;   // keys per tile
  static constexpr int NT = KT / 32;             // 32-key N-tiles per tile
  static constexpr int TileB = KT * 128;         // bytes of a tile
  static constexpr int Loads = KL + 1;           // loads per wave per tile: keys, scales
  static_assert((S & (S - 1)) == 0, "ring depth is a power of two");
};


// Store v at base + off on the lanes set in `mask` (a subset of the active
// lanes), without a branch: exec is narrowed around the one store and
// restored.  base is uniform (scalar registers), off a per-lane byte offset.
// Nothing in the kernel reads the stored memory, hence no memory clobber.
__device__ __forceinline__ void store_lanes(const float* base, uint32_t off, float v, uint64_t mask) {
  uint64_t saved;
  asm volatile(
      "s_mov_b64 %0, exec\n\ts_mov_b64 exec, %4\n\tglobal_store_dword %1, %2, %3\n\ts_mov_b64 exec, %0"
      : "=&s"(saved)
      : "v"(off), "v"(v), "s"(base), "s"(mask));
}

__device__ __forceinline__ f32x16 mfma_f8(const i32x8& a, const i32x8& b, const f32x16& c) {
  // cbsz = blgp = 0: both operands e4m3; scale exponents 127 = 2^0
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

template <int KL, int S>
__global__ __launch_bounds__(64 * kF8Waves, 1) void idx_score_h64_fp8_kernel(
    const uint8_t* __restrict__ q8, const float* __restrict__ q_scale, const float* __restrict__ w,
    int64_t w_stride, const uint8_t* __restrict__ k8, const float* __restrict__ k_scale,
    const int32_t* __restrict__ q_pos, int n_q, int n_k, float* __restrict__ scores, int64_t ld,
    int n_qblocks, int n_chunks, int chunk_keys) {
  constexpr int H = 64, DI = 128;
  using G = F8Geom<KL, S>;
  constexpr int kF8KT = G::KT, kF8NT = G::NT, kF8Stages = S, kF8Loads = G::Loads;
  __shared__ __attribute__((aligned(1024))) uint8_t s_k[S][G::TileB];
  __shared__ __attribute__((aligned(16))) float s_sc[S][G::KT];
  __shared__ int s_pos[kF8Waves], s_qid[kF8Waves], s_allpos[64 * kF8Waves];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qb = n_qblocks - 1 - (int)(blockIdx.x / n_chunks);
  const int chunk = (int)(blockIdx.x % n_chunks);
  const int q0 = qb * kF8Waves;
  idx_block_queries<kF8Waves>(q_pos, n_q, n_k, q0, s_qid, s_pos, s_allpos);
  int pmax = -1;
#pragma unroll
  for (int t = 0; t < kF8Waves; ++t) pmax = max(pmax, s_pos[t]);
  const int k_begin = chunk * chunk_keys;
  const int k_end = min(k_begin + chunk_keys, pmax + 1);
  if (k_begin >= k_end) return;   // uniform across the workgroup
  const int ntiles = (k_end - k_begin + kF8KT - 1) / kF8KT;
  // the wave's query: position (scalar), row (clamped for the operand reads)
  const int mypos = __builtin_amdgcn_readfirstlane(s_pos[wave]);
  const int myq = __builtin_amdgcn_readfirstlane(s_qid[wave]);   // -1: no query in this slot
  const bool q_ok = myq >= 0;
  const int qi = q_ok ? myq : 0;

  // ---- A operands: head row 32t + lrow, bytes 64j + 32 khalf .. +31 ----
  const int lrow = lane & 31, khalf = lane >> 5;
  i32x8 a[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const u32x4* src = reinterpret_cast<const u32x4*>(q8 + ((int64_t)qi * H + 32 * t + lrow) * DI + 64 * j +
                                                        32 * khalf);
      const u32x4 lo = src[0], hi = src[1];
      a[t][j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2],
                      (int)hi[3]};
    }
  // head weight times the head row's scale, for accumulator rows
  // 32t + 8(jj>>2) + 4khalf + (jj&3)
  float wv[2][16];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      const int h = 32 * t + 8 * (jj >> 2) + 4 * khalf + (jj & 3);
      wv[t][jj] = w[(int64_t)qi * w_stride + h] * q_scale[(int64_t)qi * H + h];
    }

  // ---- gather of tile i (keys k_begin + 96i ..) into slot i % kF8Stages ----
  const int dkey = 8 * KL * wave + (lane >> 3);   // this lane's key within the tile, load 0
  auto issue = [&](int i) {
    const int slot = i & (S - 1);
    const int kt = k_begin + kF8KT * i;
    const uint32_t dst = (uint32_t)(uintptr_t)(idx_lds_u8*)&s_k[slot][1024 * KL * wave];
#pragma unroll
    for (int j = 0; j < KL; ++j)   // keys 8j apart share (key >> 1) & 7's parity pattern: 8j >> 1 = 4j
      idx_dma16(k8 + (int64_t)min(kt + dkey + 8 * j, n_k - 1) * DI + 16 * ((lane & 7) ^ (((dkey + 8 * j) >> 1) & 7)),
                dst + 1024 * j);
    const uint32_t sdst =
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)&s_sc[slot][8 * KL * wave];
    if (lane < 8 * KL) idx_dma4(k_scale + min(kt + 8 * KL * wave + lane, n_k - 1), sdst);
  };
  idx_wait_vmcnt<0>();   // operand loads retired: only gathers are outstanding below
#pragma unroll
  for (int i = 0; i < kF8Stages - 1; ++i) issue(i);

  // B operand of N-tile u, k-step j: key 32u + lrow, chunks 4j + 2khalf and
  // 4j + 2khalf + 1 at their swizzled slots ((key >> 1) & 7 = (lrow >> 1) & 7).
  int boff[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) boff[j][h] = lrow * 128 + 16 * ((4 * j + 2 * khalf + h) ^ ((lrow >> 1) & 7));

  // ReLU, head weights, sum over the lane's 32 head rows and the other 32
  // held by the lane 32 apart; times the key scale.  Both halves end with
  // the head sum of key column lrow.
  auto head_sum = [&](const f32x16& c0, const f32x16& c1, float sc) {
    float part = 0.f;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) {
      part = fmaf(wv[0][jj], __int_as_float(max(__float_as_int(c0[jj]), 0)), part);
      part = fmaf(wv[1][jj], __int_as_float(max(__float_as_int(c1[jj]), 0)), part);
    }
    part += __uint_as_float(__builtin_amdgcn_permlane32_swap(__float_as_uint(part), __float_as_uint(part), false,
                                                             false)[1]);
    return part * sc;
  };
  // keys key0 .. key0 + 31 of the wave's row, from the lower half's lanes,
  // up to the query's position; base and mask are scalar
  const float* row = scores + (int64_t)qi * ld;
  const uint32_t lane_off = 4u * (uint32_t)lrow;
  auto store = [&](float v, int key0) {
    const int nv = q_ok ? min(max(mypos - key0 + 1, 0), 32) : 0;
    const uint64_t m = nv >= 32 ? 0xFFFFFFFFull : ((1ull << nv) - 1);
    store_lanes(row + key0, lane_off, v, m);
  };
  // B operands and the key scale are read one N-tile ahead of their MFMAs,
  // so the last N-tile of tile i reads tile i + 1: the waits cover tiles i
  // and i + 1, leaving kF8Stages - 3 tiles in flight.
  idx_wait_vmcnt<(kF8Stages - 2) * kF8Loads>();
  idx_sync_lds();
  u32x4 bn[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int h = 0; h < 2; ++h) bn[j][h] = *reinterpret_cast<const u32x4*>(s_k[0] + boff[j][h]);
  float scn = s_sc[0][lrow];
  // Each N-tile's MFMAs are followed by its own epilogue; the three waves of
  // a SIMD overlap one wave's MFMAs with another's epilogue.  A tile's sums
  // are stored at the top of the next iteration, beside the wait, barrier
  // and loads, so that the N-tile loop is one scheduling region.
  float res[kF8NT];
  for (int i = 0; i < ntiles; ++i) {
    const int k0 = k_begin + kF8KT * i;
    if (i > 0) {
#pragma unroll
      for (int u = 0; u < kF8NT; ++u) store(res[u], k0 - kF8KT + 32 * u);
    }
    idx_wait_vmcnt<(kF8Stages - 3) * kF8Loads>();
    idx_sync_lds();             // for every wave; slot (i - 1) % S is free
    issue(i + kF8Stages - 1);   // past the range these load clamped keys into a free slot
    const uint8_t* tile = s_k[i & (S - 1)];
#pragma unroll
    for (int u = 0; u < kF8NT; ++u) {
      const bool last = u + 1 == kF8NT;
      const int nslot = (last ? i + 1 : i) & (S - 1);
      const uint8_t* nxt = last ? s_k[nslot] : tile + 4096 * (u + 1);
      const float* nsc = &s_sc[nslot][last ? 0 : 32 * (u + 1)];
      const float sc = scn;
      f32x16 c0 = f32x16{}, c1 = f32x16{};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 lo = bn[j][0], hi = bn[j][1];
        const i32x8 b = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2],
                              (int)hi[3]};
        bn[j][0] = *reinterpret_cast<const u32x4*>(nxt + boff[j][0]);
        bn[j][1] = *reinterpret_cast<const u32x4*>(nxt + boff[j][1]);
        c0 = mfma_f8(a[0][j], b, c0);
        c1 = mfma_f8(a[1][j], b, c1);
      }
      scn = nsc[lrow];
      res[u] = head_sum(c0, c1, sc);
    }
  }
#pragma unroll
  for (int u = 0; u < kF8NT; ++u) store(res[u], k_begin + kF8KT * (ntiles - 1) + 32 * u);
  idx_wait_vmcnt<0>();   // no load may land in LDS after the workgroup has left
}

template <int KL, int S>
static hipError_t launch_f8(const IdxArgs& A, hipStream_t st) {
  constexpr int KT = F8Geom<KL, S>::KT;
  const int n_qblocks = (A.n_q + kF8Waves - 1) / kF8Waves;
  int n_chunks = 1;
  const int target_wgs = 1024;
  if (n_qblocks < target_wgs) n_chunks = (target_wgs + n_qblocks - 1) / n_qblocks;
  int chunk_keys = (int)((A.n_k + n_chunks - 1) / n_chunks);
  chunk_keys = ((chunk_keys + KT - 1) / KT) * KT;
  if (chunk_keys < 4 * KT) chunk_keys = 4 * KT;
  n_chunks = (int)((A.n_k + chunk_keys - 1) / chunk_keys);
  const long long grid = (long long)n_qblocks * n_chunks;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((idx_score_h64_fp8_kernel<KL, S>), dim3((unsigned)grid), dim3(64 * kF8Waves), 0, st,
                     static_cast<const uint8_t*>(A.q_idx), A.q_scale, A.w, A.w_stride,
                     static_cast<const uint8_t*>(A.k_idx), A.k_scale, A.q_pos, A.n_q, (int)A.n_k, A.scores, A.ld,
                     n_qblocks, n_chunks, chunk_keys);
  return hipGetLastError();
}

hipError_t launch_index_scores_fp8(const IdxArgs& A, hipStream_t st) {
  if (A.h_idx != 64 || A.d_idx != 128 || !A.fp8 || !A.q_scale) return hipErrorInvalidValue;
  return launch_f8<1, 8>(A, st);   // 96-key tiles, 8 in the ring (~99 KiB of LDS)
}

hipError_t launch_index_scores(const IdxArgs& A, hipStream_t st) {
  const bool f8 = A.fp8;
  if (A.q_scale) return launch_index_scores_fp8(A, st);
  if (A.h_idx == 64 && A.d_idx == 128) return f8 ? launch_idx_h64_f8k(A, st) : launch_idx_h64(A, st);
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
