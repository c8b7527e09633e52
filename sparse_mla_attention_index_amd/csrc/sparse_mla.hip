// Sparse MLA gather-attention kernel (gfx950), absorbed / "MQA" mode.
//
// All 64 heads of one query attend over the query's selected latent rows:
// z = tau * q_h . kv_s[0:576], softmax over the selected set, o_h = sum_s
// p_s kv_s[0:512] (GLM-5.3 part 2, "PCP : répartir les tokens, pas les
// têtes" and footnote 1: one KV row read serves every head; QK over 576, PV
// over 512).
//
// One workgroup (4 waves) per query; wave w owns heads 16w..16w+15.  The
// selected rows are gathered 32 at a time into a double-buffered, row-major
// LDS tile that serves both products:
//   S^T[row][head] = K_tile . Q^T    v_mfma_f32_16x16x32_bf16, A = K rows read
//                                    with ds_read_b128, B = the wave's Q
//                                    fragment kept in registers;
//   O^T[dim][head] += V^T . P^T      A = V^T read straight from the row-major
//                                    tile with ds_read_b64_tr_b16, B = P taken
//                                    from the S^T accumulators in registers.
// Writing the products transposed puts one head per lane column in both
// accumulators, so the online-softmax statistics of a head and the output
// rows they rescale live in the same lanes, and P never leaves registers.
// Softmax runs in fp32 in the exp2 domain with a running max; the rescale of
// O is skipped when no head's max moved.
#include "sma_device.h"
#include "sma_launch.h"

namespace sma {

constexpr int kMlaRows = 32;                // gathered rows per tile
constexpr int kMlaRowB = kDqk * 2 + 16;     // padded LDS row, bytes (1168)
constexpr int kMlaThreads = 256;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

template <bool FP8, bool OUT_F32>
__global__ __launch_bounds__(kMlaThreads, 1) void sparse_mla_kernel(
    const uint16_t* __restrict__ q, const void* __restrict__ kv, const float* __restrict__ kv_scale,
    int n_k, const int32_t* __restrict__ idx, int n_q, int K, float scale_log2,
    void* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) uint8_t s_kv[2][kMlaRows * kMlaRowB];
  __shared__ int s_list[SMA_MAX_TOPK_DEV];
  __shared__ float s_scale[2][kMlaRows];
  __shared__ uint32_t s_cnt[kMlaThreads / 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qi = blockIdx.x;
  const int g = lane >> 4, i = lane & 15;   // lane group (k slot) and column (head)

  // ---- compact the valid indices, keeping their order ----
  constexpr int PER = SMA_MAX_TOPK_DEV / kMlaThreads;   // 8
  int v[PER];
  uint32_t cnt = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int j = tid * PER + e;
    int x = j < K ? idx[(int64_t)qi * K + j] : -1;
    if (x < 0 || x >= n_k) x = -1;
    v[e] = x;
    cnt += x >= 0;
  }
  uint32_t incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) s_cnt[wave] = incl;
  __syncthreads();
  uint32_t before = incl - cnt, total = 0;
#pragma unroll
  for (int w = 0; w < kMlaThreads / 64; ++w) {
    if (w < wave) before += s_cnt[w];
    total += s_cnt[w];
  }
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if (v[e] >= 0) s_list[before++] = v[e];
  __syncthreads();
  const int n_valid = (int)total;

  const int head = 16 * wave + i;
  if (n_valid == 0) {
    for (int mt = 0; mt < kDv / 16; ++mt) {
      const int64_t o_off = ((int64_t)qi * kHeads + head) * kDv + 16 * mt + 4 * g;
      if constexpr (OUT_F32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + o_off) = f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + o_off) = u32x2{0u, 0u};
      }
    }
    if (lse && g == 0) lse[(int64_t)qi * kHeads + head] = -INFINITY;
    return;
  }

  // ---- the wave's Q fragment: head 16w+i, dims 32ks + 8g .. +7 ----
  bf16x8 qf[kDqk / 32];
  {
    const uint16_t* src = q + ((int64_t)qi * kHeads + head) * kDqk + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kDqk / 32; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(src + 32 * ks);
  }

  // ---- gather staging ----
  constexpr int NCH = FP8 ? (kMlaRows * kDqk / 16 + kMlaThreads - 1) / kMlaThreads
                          : kMlaRows * kDqk / 8 / kMlaThreads;   // 16-byte loads per thread
  u32x4 stage[NCH];
  float stage_sc = 0.f;
  auto load_tile = [&](int t) {
    const int r0 = t * kMlaRows;
#pragma unroll
    for (int r = 0; r < NCH; ++r) {
      const int c = tid + kMlaThreads * r;
      if constexpr (FP8) {
        if (c < kMlaRows * kDqk / 16) {
          const int row = c / (kDqk / 16), col = c % (kDqk / 16);
          const int li = r0 + row < n_valid ? r0 + row : 0;
          stage[r] = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(kv) +
                                                     (int64_t)s_list[li] * kDqk + col * 16);
        }
      } else {
        const int row = c / (kDqk / 8), col = c % (kDqk / 8);
        const int li = r0 + row < n_valid ? r0 + row : 0;
        stage[r] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(kv) +
                                                   (int64_t)s_list[li] * kDqk + col * 8);
      }
    }
    if constexpr (FP8) {
      if (tid < kMlaRows) {
        const int li = r0 + tid < n_valid ? r0 + tid : 0;
        stage_sc = kv_scale[s_list[li]];
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int r = 0; r < NCH; ++r) {
      const int c = tid + kMlaThreads * r;
      if constexpr (FP8) {
        if (c < kMlaRows * kDqk / 16) {
          const int row = c / (kDqk / 16), col = c % (kDqk / 16);
          uint8_t* dst = &s_kv[buf][row * kMlaRowB + col * 32];
          const u32x2 t0 = e4m3x4_to_bf16x4(stage[r][0]), t1 = e4m3x4_to_bf16x4(stage[r][1]);
          const u32x2 t2 = e4m3x4_to_bf16x4(stage[r][2]), t3 = e4m3x4_to_bf16x4(stage[r][3]);
          *reinterpret_cast<u32x4*>(dst) = u32x4{t0[0], t0[1], t1[0], t1[1]};
          *reinterpret_cast<u32x4*>(dst + 16) = u32x4{t2[0], t2[1], t3[0], t3[1]};
        }
      } else {
        const int row = c / (kDqk / 8), col = c % (kDqk / 8);
        *reinterpret_cast<u32x4*>(&s_kv[buf][row * kMlaRowB + col * 16]) = stage[r];
      }
    }
    if constexpr (FP8) {
      if (tid < kMlaRows) s_scale[buf][tid] = stage_sc;
    }
  };

  // ---- running state: O^T[dim 16mt+4g+r][head i] in o[mt][r] ----
  f32x4 o[kDv / 16];
#pragma unroll
  for (int mt = 0; mt < kDv / 16; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;   // running max of the head's logits (log2 domain)
  float l_run = 0.f;         // this lane's share of the softmax denominator

  const int ntiles = (n_valid + kMlaRows - 1) / kMlaRows;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    const bool has_next = t + 1 < ntiles;
    if (has_next) load_tile(t + 1);
    const uint8_t* tile = s_kv[buf];

    // S^T = K . Q^T : rows 16mt + 4g + r, head i
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < kDqk / 32; ++ks) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(tile + (16 * mt + i) * kMlaRowB + (32 * ks + 8 * g) * 2);
        sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], sacc[mt], 0, 0, 0);
      }
    }

    // online softmax (log2 domain)
    const int valid_rows = n_valid - t * kMlaRows;
    float s2[8];
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * mt + 4 * g + r;
        float x = sacc[mt][r] * scale_log2;
        if constexpr (FP8) x *= s_scale[buf][row];
        x = row < valid_rows ? x : -INFINITY;
        s2[4 * mt + r] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    float psum = 0.f;
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pe = exp2f(s2[e] - m_new);
      psum += pe;
      pv[e] = pe;
      if constexpr (FP8) pv[e] = pe * s_scale[buf][16 * (e / 4) + 4 * g + (e % 4)];
    }
    l_run = l_run * alpha + psum;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int mt = 0; mt < kDv / 16; ++mt) o[mt] *= alpha;
    }
    m_run = m_new;
    bf16x8 pb;
#pragma unroll
    for (int e = 0; e < 8; ++e) pb[e] = (__bf16)pv[e];

    // O^T += V^T . P^T ; V^T columns read transposed from the row-major tile
    const uint8_t* va_base = tile + (4 * g + (i >> 2)) * kMlaRowB + 8 * (i & 3);
    const uint8_t* vb_base = va_base + 16 * kMlaRowB;
#pragma unroll
    for (int mt = 0; mt < kDv / 16; ++mt) {
      const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(va_base + 32 * mt));
      const i16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vb_base + 32 * mt));
      const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
      o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, o[mt], 0, 0, 0);
    }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- normalise and write ----
  float l_tot = l_run + __shfl_xor(l_run, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  const float inv = 1.f / l_tot;
#pragma unroll
  for (int mt = 0; mt < kDv / 16; ++mt) {
    const int64_t o_off = ((int64_t)qi * kHeads + head) * kDv + 16 * mt + 4 * g;
    const f32x4 r = o[mt] * inv;
    if constexpr (OUT_F32) {
      *reinterpret_cast<f32x4*>(static_cast<float*>(out) + o_off) = r;
    } else {
      *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + o_off) =
          u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
    }
  }
  if (lse && g == 0)
    lse[(int64_t)qi * kHeads + head] = (m_run + __log2f(l_tot)) * 0.69314718055994531f;
}

// ---------------------------------------------------------------------------
// bf16 KV: the same computation with the gather issued as direct
// global->LDS loads (global_load_lds_dwordx4) into a 4-deep ring of 32-row
// tiles, so three tiles are in flight while one is consumed and no VGPRs
// stage the gather.  Tiles are unpadded (1152 B per row) and every wave
// issues exactly 9 one-KiB loads per tile, which keeps the per-wave vmcnt
// bookkeeping exact.  Inside a row the 16-byte chunks are XOR-swizzled by
// the row's low three bits so the K reads (16 rows, same chunk) and the
// transposed V reads spread over the LDS banks.
// ---------------------------------------------------------------------------
constexpr int kDmaStages = 4;
constexpr float kRefGap = 64.f;                         // log2 units
constexpr int kDmaRowB = kDqk * 2;                      // 1152
constexpr int kDmaTileB = kMlaRows * kDmaRowB;          // 36864
constexpr int kDmaLoadsPerWave = kDmaTileB / 1024 / 4;  // 9

typedef __attribute__((address_space(3))) uint8_t lds_u8;

// One 16-byte-per-lane global->LDS load: lane l's 16 bytes land at LDS byte
// address lds_base + 16*l.  Issued from inline assembly so that the
// compiler's wait-count insertion does not treat it as aliasing the ring
// slots being read; completion is tracked by hand with wait_vmcnt<>.
__device__ __forceinline__ void dma_load16(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr), "s"(lds_base)
               : "memory", "m0");
}

__device__ __forceinline__ int chunk_swz(int row, int c) { return c ^ (row & 7); }

// Place a value in the AGPR file (an empty asm with an AGPR in/out operand).
// MFMA source operands may come from AGPRs, so the wave's 72 Q registers can
// live there, leaving the VGPR file to the output accumulators and to K
// operands prefetched from LDS ahead of their MFMAs.
__device__ __forceinline__ void pin_agpr(bf16x8& x) { asm volatile("" : "+a"(x)); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that makes this wave's LDS writes visible (waits for
// its outstanding LDS operations) but leaves vector-memory loads in flight:
// the gather DMA is waited for explicitly with wait_vmcnt<>.
__device__ __forceinline__ void block_sync_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The bf16 kernel splits a query's work over its 4 waves so that each
// gathered byte is read from LDS by as few waves as possible:
//   QK   wave w computes S^T for rows 16*(w&1)..+15 of the tile and heads
//        32*(w>>1)..+31 (one K operand read feeds two 16-head MFMAs; the
//        wave's Q fragment is 32 heads x 576 dims, 144 AGPRs);
//   PV   wave w owns output dims 128w..128w+127 for all 64 heads, reading
//        only its slice of V^T (transposed LDS reads) and the tile's P,
//        which the QK waves write to LDS as bf16 [head][row].
// Per 32-row tile the CU's LDS moves 160 KB (36 KB gather, 72 KB K, 32 KB
// V, 20 KB P) instead of the 308 KB a 16-heads-per-wave split needs.
constexpr int kPRowB = 80;                              // P^T row: 32 bf16 + 16 B pad

template <bool OUT_F32>
__global__ __launch_bounds__(kMlaThreads, 1) void sparse_mla_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, int n_k,
    const int32_t* __restrict__ idx, int n_q, int K, float scale_log2, void* __restrict__ out,
    float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_kv[kDmaStages][kDmaTileB];
  __shared__ int s_list[SMA_MAX_TOPK_DEV];
  __shared__ __attribute__((aligned(16))) uint8_t s_p[kHeads * kPRowB];
  __shared__ float s_red[4][kHeads];
  __shared__ uint32_t s_cnt[kMlaThreads / 64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qi = blockIdx.x;
  const int g = lane >> 4, i = lane & 15;
  const int rh = wave & 1, hh = wave >> 1;   // QK role: row half, head half

  // ---- compact the valid indices, keeping their order ----
  constexpr int PER = SMA_MAX_TOPK_DEV / kMlaThreads;
  int v[PER];
  uint32_t cnt = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int j = tid * PER + e;
    int x = j < K ? idx[(int64_t)qi * K + j] : -1;
    if (x < 0 || x >= n_k) x = -1;
    v[e] = x;
    cnt += x >= 0;
  }
  uint32_t incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) s_cnt[tid >> 6] = incl;
  __syncthreads();
  uint32_t before = incl - cnt, total = 0;
#pragma unroll
  for (int w = 0; w < kMlaThreads / 64; ++w) {
    if (w < (tid >> 6)) before += s_cnt[w];
    total += s_cnt[w];
  }
#pragma unroll
  for (int e = 0; e < PER; ++e)
    if (v[e] >= 0) s_list[before++] = v[e];
  __syncthreads();
  const int n_valid = (int)total;

  // output element (head 16n+i, dim 128w + 16m + 4g + r) lives in o[m][n][r]
  auto out_off = [&](int m, int n) {
    return ((int64_t)qi * kHeads + 16 * n + i) * kDv + 128 * (tid >> 6) + 16 * m + 4 * g;
  };
  if (n_valid == 0) {
    for (int m = 0; m < 8; ++m)
      for (int n = 0; n < 4; ++n) {
        if constexpr (OUT_F32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(out) + out_off(m, n)) = f32x4{0.f, 0.f, 0.f, 0.f};
        } else {
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + out_off(m, n)) = u32x2{0u, 0u};
        }
      }
    if (lse && tid < kHeads) lse[(int64_t)qi * kHeads + tid] = -INFINITY;
    return;
  }

  // ---- Q fragment: heads 32hh + 16n + i, dims 32ks + 8g .. +7 ----
  bf16x8 qf[2][kDqk / 32];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const uint16_t* src = q + ((int64_t)qi * kHeads + 32 * hh + 16 * n + i) * kDqk + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kDqk / 32; ++ks) qf[n][ks] = *reinterpret_cast<const bf16x8*>(src + 32 * ks);
  }
  // Retire the Q loads here: from now on every outstanding vector-memory
  // operation of the wave is a gather DMA, which wait_vmcnt<> counts.
  wait_vmcnt<0>();
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int ks = 0; ks < kDqk / 32; ++ks) (void)qf[n][ks];

  // ---- DMA gather of tile t into ring slot b (9 one-KiB loads per wave) ----
  const uint8_t* kvb = reinterpret_cast<const uint8_t*>(kv);
  auto issue_tile = [&](int t, int b) {
    const uint8_t* src[kDmaLoadsPerWave];
#pragma unroll
    for (int j = 0; j < kDmaLoadsPerWave; ++j) {
      const int p = (wave * kDmaLoadsPerWave + j) * 1024 + lane * 16;
      const int row = p / kDmaRowB;
      const int c = chunk_swz(row, (p - row * kDmaRowB) >> 4);
      const int li = t * kMlaRows + row;
      src[j] = kvb + (int64_t)s_list[li < n_valid ? li : 0] * kDmaRowB + c * 16;
    }
#pragma unroll
    for (int j = 0; j < kDmaLoadsPerWave; ++j) {
      const uint32_t dst = (uint32_t)(uintptr_t)(lds_u8*)&s_kv[b][(wave * kDmaLoadsPerWave + j) * 1024];
      dma_load16(src[j], __builtin_amdgcn_readfirstlane(dst));
    }
  };
  const int ntiles = (n_valid + kMlaRows - 1) / kMlaRows;

  // ---- per-lane LDS byte offsets (swizzle: chunk ^= row & 7) ----
  // K operand: row 16rh + i, chunk 4ks + g.
  const int xa = i & 7;
  const int kbase = (16 * rh + i) * kDmaRowB + (((g ^ xa) & 3) << 4);
  const int kb_even = kbase + ((xa >> 2) << 6);
  const int kb_odd = kbase + ((1 - (xa >> 2)) << 6);
  // V^T operand of M-tile m: rows 8g + (i>>2) (+4), dims 128w + 16m + 4(i&3),
  // i.e. chunk 16w + 2m + vsub, 8-byte half i&1; (2(m&3)+vsub) ^ x splits per m&3.
  const int xr = i >> 2, vsub = (i & 3) >> 1, vhalf = (i & 1) * 8;
  const int ra = 8 * g + xr;
  int va_off[4], vb_off[4];
#pragma unroll
  for (int mm = 0; mm < 4; ++mm) {
    const int cl = 2 * mm + vsub;
    va_off[mm] = ra * kDmaRowB + (16 * wave + (cl ^ xr)) * 16 + vhalf;
    vb_off[mm] = (ra + 4) * kDmaRowB + (16 * wave + (cl ^ xr ^ 4)) * 16 + vhalf;
  }
  // P^T operand of N-tile n: head 16n + i, rows 8g..8g+7
  const int p_rd = i * kPRowB + 16 * g;
  // P^T written by the QK roles: head 32hh + 16n + i, rows 16rh + 4g .. +3
  const int p_wr = (32 * hh + i) * kPRowB + (16 * rh + 4 * g) * 2;

  f32x4 o[8][4];
  float m_ref[2], m_max[2] = {-INFINITY, -INFINITY}, l_part[2];   // per QK head 32hh+16n+i

  // One sweep over the selected rows with a FIXED per-head exponent
  // reference (the first tile's maximum, or the exact maximum on a rerun):
  // O is only ever touched by MFMAs in the loop.  Returns whether some logit
  // passed m_ref + kRefGap (weights above 1 are fine below that).
  auto sweep = [&](bool ref_from_first_tile) -> bool {
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) o[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_part[0] = l_part[1] = 0.f;
    bool far = false;
#pragma unroll
    for (int t = 0; t < kDmaStages - 1; ++t)
      if (t < ntiles) issue_tile(t, t);

    for (int t = 0; t < ntiles; ++t) {
      const int ahead = min(kDmaStages - 2, ntiles - 1 - t);
      if (ahead >= 2) wait_vmcnt<2 * kDmaLoadsPerWave>();
      else if (ahead == 1) wait_vmcnt<kDmaLoadsPerWave>();
      else wait_vmcnt<0>();
      block_sync_lds();   // tile t in LDS; every wave is done with tile t-1 and P
      if (t + kDmaStages - 1 < ntiles) issue_tile(t + kDmaStages - 1, (t + kDmaStages - 1) % kDmaStages);
      const uint8_t* tile = s_kv[t % kDmaStages];

      // ---- S^T (16 rows x 32 heads) = K . Q^T ----
      constexpr int kKs = kDqk / 32, kPf = 6;
      auto kread = [&](int ks) {
        return *reinterpret_cast<const bf16x8*>(tile + ((ks & 1) ? kb_odd : kb_even) + (ks >> 1) * 128);
      };
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      bf16x8 kop[kPf];
#pragma unroll
      for (int ks = 0; ks < kPf; ++ks) kop[ks] = kread(ks);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) {
        const bf16x8 a = kop[ks % kPf];
        if (ks + kPf < kKs) kop[ks % kPf] = kread(ks + kPf);
        sacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[0][ks], sacc[0], 0, 0, 0);
        sacc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[1][ks], sacc[1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }

      // ---- softmax weights with the fixed reference ----
      const int valid_rows = n_valid - t * kMlaRows;
      float s2[2][4], mx[2];
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        mx[n] = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float x = 16 * rh + 4 * g + r < valid_rows ? sacc[n][r] * scale_log2 : -INFINITY;
          s2[n][r] = x;
          mx[n] = fmaxf(mx[n], x);
        }
      }
      if (ref_from_first_tile && t == 0) {
        // reference = max over the first tile's 32 rows (both row halves)
#pragma unroll
        for (int n = 0; n < 2; ++n) {
          float x = fmaxf(mx[n], __shfl_xor(mx[n], 16, 64));
          x = fmaxf(x, __shfl_xor(x, 32, 64));
          if (g == 0) s_red[wave][16 * n + i] = x;
        }
        block_sync_lds();
#pragma unroll
        for (int n = 0; n < 2; ++n) m_ref[n] = fmaxf(s_red[wave][16 * n + i], s_red[wave ^ 1][16 * n + i]);
      }
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        m_max[n] = fmaxf(m_max[n], mx[n]);
        far |= mx[n] > m_ref[n] + kRefGap;
        float ps = 0.f;
        float pe[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pe[r] = __builtin_amdgcn_exp2f(fminf(s2[n][r] - m_ref[n], kRefGap));
          ps += pe[r];
        }
        l_part[n] += ps;
        *reinterpret_cast<u32x2*>(s_p + p_wr + 16 * n * kPRowB) =
            u32x2{pack_bf16x2(pe[0], pe[1]), pack_bf16x2(pe[2], pe[3])};
      }
      block_sync_lds();   // P of tile t complete

      // ---- O^T (128 dims x 64 heads) += V^T . P^T ----
      bf16x8 pb[4];
#pragma unroll
      for (int n = 0; n < 4; ++n)
        pb[n] = *reinterpret_cast<const bf16x8*>(s_p + p_rd + 16 * n * kPRowB);
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const int mo = (m >> 2) * 128;
        const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + va_off[m & 3] + mo));
        const i16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + vb_off[m & 3] + mo));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int n = 0; n < 4; ++n) o[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[n], o[m][n], 0, 0, 0);
      }
    }
    return far;
  };

  // Combine per-wave partials over the two row halves: per QK head, the
  // maximum (op = max) or the sum (op = add) of the lanes' values.
  auto combine_heads = [&](float (&vals)[2], bool is_max) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      float x = vals[n];
      const float y = __shfl_xor(x, 16, 64);
      x = is_max ? fmaxf(x, y) : x + y;
      const float z = __shfl_xor(x, 32, 64);
      x = is_max ? fmaxf(x, z) : x + z;
      if (g == 0) s_red[wave][16 * n + i] = x;
    }
    block_sync_lds();
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const float a = s_red[wave][16 * n + i], b = s_red[wave ^ 1][16 * n + i];
      vals[n] = is_max ? fmaxf(a, b) : a + b;
    }
    block_sync_lds();
  };

  const bool far = sweep(true);
  if (lane == 0) s_cnt[tid >> 6] = far ? 1u : 0u;
  block_sync_lds();
  const bool redo = (s_cnt[0] | s_cnt[1] | s_cnt[2] | s_cnt[3]) != 0u;
  if (redo) {
    combine_heads(m_max, true);
    m_ref[0] = m_max[0];
    m_ref[1] = m_max[1];
    sweep(false);
  }
  combine_heads(l_part, false);   // l per QK head (32hh + 16n + i), all rows

  // every wave needs l for all 64 heads: publish by head
  if (rh == 0 && g == 0) {
    s_red[2][32 * hh + i] = l_part[0];
    s_red[2][32 * hh + 16 + i] = l_part[1];
    s_red[3][32 * hh + i] = m_ref[0];
    s_red[3][32 * hh + 16 + i] = m_ref[1];
  }
  block_sync_lds();
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const float inv = 1.f / s_red[2][16 * n + i];
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const f32x4 r = o[m][n] * inv;
      if constexpr (OUT_F32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + out_off(m, n)) = r;
      } else {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + out_off(m, n)) =
            u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
      }
    }
  }
  if (lse && tid < kHeads)
    lse[(int64_t)qi * kHeads + tid] = (s_red[3][tid] + __log2f(s_red[2][tid])) * 0.69314718055994531f;
}

hipError_t launch_sparse_mla(const MlaArgs& A, hipStream_t st) {
  if (A.n_q <= 0) return hipSuccess;
  const float scale_log2 = A.sm_scale * 1.4426950408889634f;
  const dim3 grid((unsigned)A.n_q), block(kMlaThreads);
  if (A.fp8) {
    if (A.out_f32)
      hipLaunchKernelGGL((sparse_mla_kernel<true, true>), grid, block, 0, st, A.q, A.kv, A.kv_scale, (int)A.n_k,
                         A.idx, A.n_q, A.top_k, scale_log2, A.out, A.lse);
    else
      hipLaunchKernelGGL((sparse_mla_kernel<true, false>), grid, block, 0, st, A.q, A.kv, A.kv_scale,
                         (int)A.n_k, A.idx, A.n_q, A.top_k, scale_log2, A.out, A.lse);
  } else {
    const uint16_t* kv = static_cast<const uint16_t*>(A.kv);
    if (A.out_f32)
      hipLaunchKernelGGL((sparse_mla_bf16_kernel<true>), grid, block, 0, st, A.q, kv, (int)A.n_k, A.idx, A.n_q,
                         A.top_k, scale_log2, A.out, A.lse);
    else
      hipLaunchKernelGGL((sparse_mla_bf16_kernel<false>), grid, block, 0, st, A.q, kv, (int)A.n_k, A.idx,
                         A.n_q, A.top_k, scale_log2, A.out, A.lse);
  }
  return hipGetLastError();
}

}  // namespace sma
