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

__device__ __forceinline__ void block_sync_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <bool OUT_F32>
__global__ __launch_bounds__(kMlaThreads, 1) void sparse_mla_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, int n_k,
    const int32_t* __restrict__ idx, int n_q, int K, float scale_log2, void* __restrict__ out,
    float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) uint8_t s_kv[kDmaStages][kDmaTileB];
  __shared__ int s_list[SMA_MAX_TOPK_DEV];
  __shared__ uint32_t s_cnt[kMlaThreads / 64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qi = blockIdx.x;
  const int g = lane >> 4, i = lane & 15;

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

  const int head = 16 * (tid >> 6) + i;
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
  // Retire the Q loads here: from now on every outstanding vector-memory
  // operation of the wave is a gather DMA, which wait_vmcnt<> counts.
  wait_vmcnt<0>();
#pragma unroll
  for (int ks = 0; ks < kDqk / 32; ++ks) pin_agpr(qf[ks]);

  // ---- DMA gather of tile t into ring slot b (9 one-KiB loads per wave) ----
  const uint8_t* kvb = reinterpret_cast<const uint8_t*>(kv);
  auto issue_tile = [&](int t, int b) {
    // all source addresses first (one round of LDS reads), then the loads
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

  // Per-lane LDS byte offsets inside a tile.  The swizzle XORs the chunk
  // index c with (row & 7); splitting c into bit fields turns every read
  // address into one of a few per-lane bases plus a compile-time offset.
  //  K reads, row 16mt+i, chunk 4ks+g:  (4ks+g)^x = 8(ks>>1) + 4((ks&1)^(x>>2)) + ((g^x)&3)
  const int xa = i & 7;
  const int kbase = i * kDmaRowB + (((g ^ xa) & 3) << 4);
  const int kb_even = kbase + ((xa >> 2) << 6);          // ks even
  const int kb_odd = kbase + ((1 - (xa >> 2)) << 6);     // ks odd
  //  V reads, rows rv and rv+16, chunk 2mt+vsub, 8-byte half vhalf:
  //  (2mt+vsub)^x = 8(mt>>2) + 2((mt&3)^(x>>1)) + (vsub^(x&1))
  const int rv = 4 * g + (i >> 2);
  const int xv = rv & 7;
  const int vsub = (i & 3) >> 1, vhalf = (i & 1) * 8;
  int vbase[4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
    vbase[m] = rv * kDmaRowB + vhalf + ((2 * (m ^ (xv >> 1)) + (vsub ^ (xv & 1))) << 4);

  // One sweep over the selected rows.  Softmax weights are exp2(z - m_ref)
  // with a FIXED per-head reference: the first tile's maximum (fast sweep)
  // or the exact maximum (rerun).  O is therefore never rescaled and is only
  // ever touched by MFMAs inside the loop.  Weights above 1 are fine up to
  // 2^kRefGap; the sweep records the true maximum m_max, and reports whether
  // any logit passed m_ref + kRefGap (then the caller reruns with m_max).
  f32x4 o[kDv / 16];
  float l_run = 0.f, m_ref = 0.f, m_max = -INFINITY;
  auto sweep = [&](bool ref_from_first_tile) -> bool {
#pragma unroll
    for (int mt = 0; mt < kDv / 16; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    l_run = 0.f;
    bool far = false;
#pragma unroll
    for (int t = 0; t < kDmaStages - 1; ++t)
      if (t < ntiles) issue_tile(t, t);

    for (int t = 0; t < ntiles; ++t) {
      // tile t is complete once at most (tiles issued after it) x 9 loads remain
      const int ahead = min(kDmaStages - 2, ntiles - 1 - t);
      if (ahead >= 2) wait_vmcnt<2 * kDmaLoadsPerWave>();
      else if (ahead == 1) wait_vmcnt<kDmaLoadsPerWave>();
      else wait_vmcnt<0>();
      block_sync_lds();
      if (t + kDmaStages - 1 < ntiles) issue_tile(t + kDmaStages - 1, (t + kDmaStages - 1) % kDmaStages);
      const uint8_t* tile = s_kv[t % kDmaStages];

      // S^T = K . Q^T : rows 16mt + 4g + r, head i.  K operands are read kPf
      // k-steps ahead of the MFMAs that consume them.
      constexpr int kKs = kDqk / 32, kPf = 4;
      auto kread = [&](int ks, int mt) {
        return *reinterpret_cast<const bf16x8*>(tile + ((ks & 1) ? kb_odd : kb_even) + (ks >> 1) * 128 +
                                               mt * 16 * kDmaRowB);
      };
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      bf16x8 kop[kPf][2];
#pragma unroll
      for (int ks = 0; ks < kPf; ++ks) {
        kop[ks][0] = kread(ks, 0);
        kop[ks][1] = kread(ks, 1);
      }
      __builtin_amdgcn_sched_barrier(0);   // keep the issue order written here
#pragma unroll
      for (int ks = 0; ks < kKs; ++ks) {
        const bf16x8 a0 = kop[ks % kPf][0], a1 = kop[ks % kPf][1];
        if (ks + kPf < kKs) {
          kop[ks % kPf][0] = kread(ks + kPf, 0);
          kop[ks % kPf][1] = kread(ks + kPf, 1);
        }
        sacc[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[ks], sacc[0], 0, 0, 0);
        sacc[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[ks], sacc[1], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }

      const int valid_rows = n_valid - t * kMlaRows;
      float s2[8];
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * mt + 4 * g + r;
          const float x = row < valid_rows ? sacc[mt][r] * scale_log2 : -INFINITY;
          s2[4 * mt + r] = x;
          mx = fmaxf(mx, x);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if (ref_from_first_tile && t == 0) m_ref = mx;
      m_max = fmaxf(m_max, mx);
      far |= mx > m_ref + kRefGap;
      float psum = 0.f;
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = __builtin_amdgcn_exp2f(fminf(s2[e] - m_ref, kRefGap));
        psum += pe;
        pb[e] = (__bf16)pe;
      }
      l_run += psum;

      // O^T += V^T . P^T ; V^T read transposed from the swizzled row-major tile
#pragma unroll
      for (int mt = 0; mt < kDv / 16; ++mt) {
        const uint8_t* vp = tile + vbase[mt & 3] + (mt >> 2) * 128;
        const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)vp);
        const i16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(vp + 16 * kDmaRowB));
        const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(va, vb, 0, 1, 2, 3, 4, 5, 6, 7));
        o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, o[mt], 0, 0, 0);
      }
    }
    return far;
  };

  // Fast sweep; a query whose logits rose more than 2^kRefGap above its first
  // tile's maximum is swept again with the exact maximum as the reference.
  // The decision is made for the whole workgroup (the gather ring is shared).
  const bool far = sweep(true);
  if (lane == 0) s_cnt[tid >> 6] = far ? 1u : 0u;
  block_sync_lds();
  const bool redo = (s_cnt[0] | s_cnt[1] | s_cnt[2] | s_cnt[3]) != 0u;
  if (redo) {
    m_ref = m_max;
    block_sync_lds();   // all waves have read the flags before the ring is reused
    sweep(false);
  }
  const float m_run = m_ref;

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
