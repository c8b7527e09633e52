// Per-head batched products of absorbed MLA (gfx950): kv_b_proj split into
// its key half W_UK and value half W_UV, each applied as a batched matrix
// product (DeepSeek multi-node page, "Couche MLA"; decode absorbs the
// matrices, "Travaux futurs"):
//   absorb_q:     q_lat[i,h,:] = W_UK[h]^T q_nope[i,h,:]   (K = 128, N = 512)
//   project_out:  o[i,h,:]     = W_UV[h]   o_lat[i,h,:]    (K = 512, N = 128)
// with W_UK[h], W_UV[h] stored [128, 512] as in kv_b_proj.
//
// One kernel: C_h = A_h . B_h over bf16 with fp32 accumulation, B given
// either K-contiguous ([N][K], W_UV) or N-contiguous ([K][N], W_UK).  A
// 256-thread workgroup computes a 128 x 128 tile of one head, four waves of
// 64 x 64 (2 x 2 v_mfma_f32_32x32x16_bf16 tiles), over 64-wide K chunks
// double-buffered in LDS.  An N-contiguous B is read with the LDS transpose
// load (ds_read_b64_tr_b16), which hands each lane four consecutive K values
// of one column.  The MFMA is issued with B as its first operand, so a lane
// holds four consecutive output columns of one row; the bf16 tile is staged
// through LDS and written back in full 256-byte row pieces.  At the 64K
// prompt both products move ~5.3 GB (the 512-wide side dominates) for
// ~0.55 TFLOP: they are bound by HBM, not by the matrix cores.
#include "sma_device.h"
#include "sma_launch.h"

namespace sma {

constexpr int kBmTM = 128, kBmTN = 128, kBmTK = 64;
constexpr int kBmThreads = 256;
constexpr int kBmRowK = kBmTK * 2 + 16;    // LDS row of a K-contiguous chunk (A, or B as [N][K]): 144 B
constexpr int kBmRowN = kBmTN * 2 + 32;    // LDS row of an N-contiguous B chunk ([K][N]): 288 B
constexpr int kBmRowC = kBmTN * 2 + 16;    // LDS row of the staged C tile: 272 B
constexpr int kBmABytes = kBmTM * kBmRowK;                 // 18,432
constexpr int kBmBBytes = kBmTN * kBmRowK;                 // 18,432 (= kBmTK * kBmRowN)
static_assert(kBmTK * kBmRowN == kBmBBytes, "both B layouts fill the same space");
static_assert(kBmTM * kBmRowC <= 2 * (kBmABytes + kBmBBytes), "C staging fits the chunk buffers");

typedef __attribute__((address_space(3))) i16x4 bm_lds_i16x4;

template <bool B_KN>
__global__ __launch_bounds__(kBmThreads, 2) void bmm_bf16_kernel(
    const uint16_t* __restrict__ A, int64_t lda, int64_t a_bs, const uint16_t* __restrict__ B, int64_t ldb,
    int64_t b_bs, uint16_t* __restrict__ C, int64_t ldc, int64_t c_bs, int M, int K, int batch, int n_tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (kBmABytes + kBmBBytes)];
  // chunk buffer b: A at b * kBmABytes, B at 2 * kBmABytes + b * kBmBBytes
  auto s_a = [&](int b) { return smem + b * kBmABytes; };
  auto s_b = [&](int b) { return smem + 2 * kBmABytes + b * kBmBBytes; };

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;         // the wave's 64 x 64 quadrant
  const int lrow = lane & 31, khalf = lane >> 5;
  // n fastest, then the head: the workgroups of one A tile run together and
  // share it in L2, and those running at once cover all heads of the same
  // rows, whose A and C rows are contiguous in memory ([token][head][...])
  const int nt = (int)(blockIdx.x % n_tiles);
  const int rest = (int)(blockIdx.x / n_tiles);
  const int h = rest % batch, mt = rest / batch;
  const int m0 = mt * kBmTM, n0 = nt * kBmTN;
  const uint16_t* Ah = A + h * a_bs;
  const uint16_t* Bh = B + h * b_bs;

  // ---- chunk staging: 16 KiB of A and of B, four 16-byte pieces each per thread ----
  u32x4 sa[4], sb[4];
  auto load_chunk = [&](int k0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = tid + kBmThreads * r;
      const int row = p >> 3, c16 = p & 7;   // A: 128 rows of 64 K
      const int mg = min(m0 + row, M - 1);
      sa[r] = *reinterpret_cast<const u32x4*>(Ah + (int64_t)mg * lda + k0 + 8 * c16);
      if constexpr (B_KN) {
        const int kr = p >> 4, n16 = p & 15;   // B: 64 K rows of 128 N
        sb[r] = *reinterpret_cast<const u32x4*>(Bh + (int64_t)(k0 + kr) * ldb + n0 + 8 * n16);
      } else {
        sb[r] = *reinterpret_cast<const u32x4*>(Bh + (int64_t)(n0 + row) * ldb + k0 + 8 * c16);
      }
    }
  };
  auto store_chunk = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = tid + kBmThreads * r;
      const int row = p >> 3, c16 = p & 7;
      *reinterpret_cast<u32x4*>(s_a(buf) + row * kBmRowK + 16 * c16) = sa[r];
      if constexpr (B_KN) {
        const int kr = p >> 4, n16 = p & 15;
        *reinterpret_cast<u32x4*>(s_b(buf) + kr * kBmRowN + 16 * n16) = sb[r];
      } else {
        *reinterpret_cast<u32x4*>(s_b(buf) + row * kBmRowK + 16 * c16) = sb[r];
      }
    }
  };

  // acc[tm][tn]: rows (of the transposed product) are output columns
  // 64wn + 32tn + 8(jj/4) + 4khalf + jj%4, the lane's column is output row
  // 64wm + 32tm + lrow
  f32x16 acc[2][2] = {{f32x16{}, f32x16{}}, {f32x16{}, f32x16{}}};
  const int nchunks = K / kBmTK;
  load_chunk(0);
  store_chunk(0);
  __syncthreads();
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    const bool has_next = c + 1 < nchunks;
    if (has_next) load_chunk((c + 1) * kBmTK);
    const uint8_t* ta = s_a(buf);
    const uint8_t* tb = s_b(buf);
#pragma unroll
    for (int ks = 0; ks < kBmTK / 16; ++ks) {
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        fa[t] = *reinterpret_cast<const bf16x8*>(ta + (64 * wm + 32 * t + lrow) * kBmRowK + (16 * ks + 8 * khalf) * 2);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        if constexpr (B_KN) {
          // lanes 16G + j: column base 16(G & 1) of the 32-column tile, K rows
          // 16ks + 8(G >> 1) + 4r + (j >> 2), columns + 4(j & 3) .. +3; lane j
          // receives column base + j (= lrow), four consecutive K rows
          const int j = lane & 15, grp = lane >> 4;
          const int col = 64 * wn + 32 * t + 16 * (grp & 1) + 4 * (j & 3);
          const int kr = 16 * ks + 8 * (grp >> 1) + (j >> 2);
          const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bm_lds_i16x4*)(tb + kr * kBmRowN + 2 * col));
          const i16x4 v1 =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((bm_lds_i16x4*)(tb + (kr + 4) * kBmRowN + 2 * col));
          fb[t] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
          fb[t] = *reinterpret_cast<const bf16x8*>(tb + (64 * wn + 32 * t + lrow) * kBmRowK + (16 * ks + 8 * khalf) * 2);
        }
      }
#pragma unroll
      for (int tm = 0; tm < 2; ++tm)
#pragma unroll
        for (int tn = 0; tn < 2; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[tn], fa[tm], acc[tm][tn], 0, 0, 0);
    }
    if (has_next) store_chunk(buf ^ 1);
    __syncthreads();
  }

  // ---- bf16 tile through LDS, then full-row 16-byte stores ----
  uint8_t* s_c = smem;
#pragma unroll
  for (int tm = 0; tm < 2; ++tm)
#pragma unroll
    for (int tn = 0; tn < 2; ++tn)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = 64 * wm + 32 * tm + lrow;
        const int col = 64 * wn + 32 * tn + 8 * q + 4 * khalf;
        const f32x16& a = acc[tm][tn];
        *reinterpret_cast<u32x2*>(s_c + row * kBmRowC + 2 * col) =
            u32x2{pack_bf16x2(a[4 * q], a[4 * q + 1]), pack_bf16x2(a[4 * q + 2], a[4 * q + 3])};
      }
  __syncthreads();
  uint16_t* Ch = C + h * c_bs;
#pragma unroll
  for (int r = 0; r < kBmTM * kBmTN / 8 / kBmThreads; ++r) {
    const int p = tid + kBmThreads * r;
    const int row = p >> 4, c16 = p & 15;
    if (m0 + row < M)
      *reinterpret_cast<u32x4*>(Ch + (int64_t)(m0 + row) * ldc + n0 + 8 * c16) =
          *reinterpret_cast<const u32x4*>(s_c + row * kBmRowC + 16 * c16);
  }
}

// K = 128 with an N-contiguous B (absorb_q): one workgroup computes every
// 128-column n-tile of its 128-row A tile.  A (both 64-wide K chunks) stays
// in LDS for the whole sweep, so it is read from memory once instead of once
// per n-tile; the next n-tile's B chunks are loaded into registers while the
// current one is multiplied, and the bf16 output tile is staged through the
// B buffers (then refilled), keeping LDS at two workgroups per CU.
__global__ __launch_bounds__(kBmThreads, 2) void bmm_k128_nsweep_kernel(
    const uint16_t* __restrict__ A, int64_t lda, int64_t a_bs, const uint16_t* __restrict__ B, int64_t ldb,
    int64_t b_bs, uint16_t* __restrict__ C, int64_t ldc, int64_t c_bs, int M, int batch, int n_tiles) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (kBmABytes + kBmBBytes)];
  auto s_a = [&](int c) { return smem + c * kBmABytes; };
  auto s_b = [&](int c) { return smem + 2 * kBmABytes + c * kBmBBytes; };
  uint8_t* s_c = smem + 2 * kBmABytes;   // the two B buffers, 36,864 bytes >= 128 x 272

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = lane & 31, khalf = lane >> 5;
  // head fastest: the workgroups running at once cover all heads of the
  // same token rows, contiguous in memory
  const int h = (int)(blockIdx.x % batch), mt = (int)(blockIdx.x / batch);
  const int m0 = mt * kBmTM;
  const uint16_t* Ah = A + h * a_bs;
  const uint16_t* Bh = B + h * b_bs;
  uint16_t* Ch = C + h * c_bs;

  u32x4 sb[2][4];
  auto load_b = [&](int n0) {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = tid + kBmThreads * r;
        const int kr = p >> 4, n16 = p & 15;
        sb[c][r] = *reinterpret_cast<const u32x4*>(Bh + (int64_t)(64 * c + kr) * ldb + n0 + 8 * n16);
      }
  };
  auto store_b = [&]() {
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = tid + kBmThreads * r;
        const int kr = p >> 4, n16 = p & 15;
        *reinterpret_cast<u32x4*>(s_b(c) + kr * kBmRowN + 16 * n16) = sb[c][r];
      }
  };
  {   // A, both K chunks, once
    u32x4 sa[2][4];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = tid + kBmThreads * r;
        const int row = p >> 3, c16 = p & 7;
        sa[c][r] = *reinterpret_cast<const u32x4*>(Ah + (int64_t)min(m0 + row, M - 1) * lda + 64 * c + 8 * c16);
      }
    load_b(0);
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = tid + kBmThreads * r;
        const int row = p >> 3, c16 = p & 7;
        *reinterpret_cast<u32x4*>(s_a(c) + row * kBmRowK + 16 * c16) = sa[c][r];
      }
    store_b();
  }
  __syncthreads();

  for (int nt = 0; nt < n_tiles; ++nt) {
    const int n0 = nt * kBmTN;
    if (nt + 1 < n_tiles) load_b(n0 + kBmTN);   // in flight during this n-tile
    f32x16 acc[2][2] = {{f32x16{}, f32x16{}}, {f32x16{}, f32x16{}}};
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint8_t* ta = s_a(c);
      const uint8_t* tb = s_b(c);
#pragma unroll
      for (int ks = 0; ks < kBmTK / 16; ++ks) {
        bf16x8 fa[2], fb[2];
#pragma unroll
        for (int t = 0; t < 2; ++t)
          fa[t] = *reinterpret_cast<const bf16x8*>(ta + (64 * wm + 32 * t + lrow) * kBmRowK + (16 * ks + 8 * khalf) * 2);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int j = lane & 15, grp = lane >> 4;
          const int col = 64 * wn + 32 * t + 16 * (grp & 1) + 4 * (j & 3);
          const int kr = 16 * ks + 8 * (grp >> 1) + (j >> 2);
          const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bm_lds_i16x4*)(tb + kr * kBmRowN + 2 * col));
          const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((bm_lds_i16x4*)(tb + (kr + 4) * kBmRowN + 2 * col));
          fb[t] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int tm = 0; tm < 2; ++tm)
#pragma unroll
          for (int tn = 0; tn < 2; ++tn)
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[tn], fa[tm], acc[tm][tn], 0, 0, 0);
      }
    }
    __syncthreads();   // every wave is done with the B buffers
#pragma unroll
    for (int tm = 0; tm < 2; ++tm)
#pragma unroll
      for (int tn = 0; tn < 2; ++tn)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int row = 64 * wm + 32 * tm + lrow;
          const int col = 64 * wn + 32 * tn + 8 * q + 4 * khalf;
          const f32x16& a = acc[tm][tn];
          *reinterpret_cast<u32x2*>(s_c + row * kBmRowC + 2 * col) =
              u32x2{pack_bf16x2(a[4 * q], a[4 * q + 1]), pack_bf16x2(a[4 * q + 2], a[4 * q + 3])};
        }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kBmTM * kBmTN / 8 / kBmThreads; ++r) {
      const int p = tid + kBmThreads * r;
      const int row = p >> 4, c16 = p & 15;
      if (m0 + row < M)
        *reinterpret_cast<u32x4*>(Ch + (int64_t)(m0 + row) * ldc + n0 + 8 * c16) =
            *reinterpret_cast<const u32x4*>(s_c + row * kBmRowC + 16 * c16);
    }
    if (nt + 1 < n_tiles) {
      __syncthreads();   // the staged tile has been read out
      store_b();
      __syncthreads();
    }
  }
}

hipError_t launch_bmm_bf16(const BmmArgs& a, hipStream_t st) {
  if (a.M <= 0 || a.batch <= 0) return hipSuccess;
  if (a.N % kBmTN || a.K % kBmTK) return hipErrorInvalidValue;
  const int m_tiles = (a.M + kBmTM - 1) / kBmTM, n_tiles = a.N / kBmTN;
  const long long grid = (long long)a.batch * m_tiles * n_tiles;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  if (a.K == 128 && a.b_kn) {
    hipLaunchKernelGGL(bmm_k128_nsweep_kernel, dim3((unsigned)(grid / n_tiles)), dim3(kBmThreads), 0, st, a.A, a.lda,
                       a.a_bs, a.B, a.ldb, a.b_bs, a.C, a.ldc, a.c_bs, a.M, a.batch, n_tiles);
    return hipGetLastError();
  }
  if (a.b_kn)
    hipLaunchKernelGGL(bmm_bf16_kernel<true>, dim3((unsigned)grid), dim3(kBmThreads), 0, st, a.A, a.lda, a.a_bs,
                       a.B, a.ldb, a.b_bs, a.C, a.ldc, a.c_bs, a.M, a.K, a.batch, n_tiles);
  else
    hipLaunchKernelGGL(bmm_bf16_kernel<false>, dim3((unsigned)grid), dim3(kBmThreads), 0, st, a.A, a.lda, a.a_bs,
                       a.B, a.ldb, a.b_bs, a.C, a.ldc, a.c_bs, a.M, a.K, a.batch, n_tiles);
  return hipGetLastError();
}

}  // namespace sma
