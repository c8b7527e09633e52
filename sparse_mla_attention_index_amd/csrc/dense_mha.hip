// Dense causal MHA prefill over the latent expanded per head (gfx950): the
// path the pages give prompts that fit inside top-k (GLM-5.3 part 2,
// "Essayez-le": without the forced MQA mode such prefill batches take dense
// MHA; DeepSeek multi-node page, "Travaux futurs": in prefill, project the
// latent into K/V space first, then run MHA; "Couche MLA": kv_b_proj's key
// and value halves).
//
//   k[s,h,:] = [W_UK[h] c_s (128), rope_s (64)]    v[s,h,:] = W_UV[h] c_s (128)
//   o[i,h,:] = sum_{s <= p_i} softmax_s(tau q[i,h,:] . k[s,h,:]) v[s,h,:]
//
// The expansion runs first as two batched bf16 products (bmm_bf16_kernel,
// the latent shared by all 64 heads, bf16 results in the workspace).  The
// attention kernel: a 256-thread workgroup takes one head and 128 queries,
// 32 per wave.  Key tiles of 32 rows (128 expanded no-rope dims + the 64
// shared rope dims, and 128 value dims; 22 KB) are staged through registers
// into double-buffered LDS and shared by the four waves.  Each wave forms
// S^T [32 keys x 32 queries] with v_mfma_f32_32x32x16_bf16 (A = K rows from
// LDS, B = its queries' Q, kept in registers), takes the online softmax per
// query column in fp32 (a lane holds 16 of a column's 32 keys, its partner
// lane + 32 the other 16), and accumulates O^T [128 dims x 32 queries] with
// A = V^T read by ds_read_b64_tr_b16 and B = P as bf16.  The key order of P
// inside each 16-key MFMA step follows the accumulator layout (a lane group
// holds keys 4g..4g+3 and 8+4g..8+4g+3), and V^T is read in that same order,
// so no register shuffle is needed between the two products.  The causal
// mask is applied per element only on tiles that reach past a wave's
// smallest query position; workgroups whose queries sit latest in the
// prompt (the longest prefixes) are dispatched first.
#include "sma_device.h"
#include "sma_launch.h"

namespace sma {

constexpr int kMhThreads = 256;                  // 4 waves
constexpr int kMhQ = 128;                        // queries per workgroup, 32 per wave
constexpr int kMhKeys = 32;                      // keys per tile
constexpr int kMhDn = 128, kMhDr = 64, kMhDqk = 192, kMhDv = 128;
constexpr int kMhRowK = kMhDqk * 2 + 16;         // 400 B: 16 consecutive rows hit distinct 16-byte slots
constexpr int kMhRowV = kMhDv * 2 + 32;          // 288 B: conflict-free transposed reads
constexpr int kMhKBytes = kMhKeys * kMhRowK;     // 12,800
constexpr int kMhVBytes = kMhKeys * kMhRowV;     //  9,216
constexpr int kMhBuf = kMhKBytes + kMhVBytes;    // 22,016

typedef __attribute__((address_space(3))) i16x4 mh_lds_i16x4;

template <bool OUT_F32>
__global__ __launch_bounds__(kMhThreads, 2) void dense_mha_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const uint16_t* __restrict__ knope,
    const uint16_t* __restrict__ vexp, const int32_t* __restrict__ q_pos, int n_q, int n_k, float scale_log2,
    void* __restrict__ out, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * kMhBuf];
  __shared__ int s_pmax[kMhThreads / 64];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, g = lane >> 5;
  const int n_qb = (n_q + kMhQ - 1) / kMhQ;
  const int h = (int)(blockIdx.x % kHeads);
  const int qb = n_qb - 1 - (int)(blockIdx.x / kHeads);   // latest queries first
  const int qi = qb * kMhQ + 32 * wave + col;              // this lane's query
  int p = -1;
  if (qi < n_q) {
    p = q_pos[qi];
    p = p < -1 ? -1 : (p > n_k - 1 ? n_k - 1 : p);
  }
  // the wave's smallest and the workgroup's largest position
  int pmin = p < 0 ? 0x7FFFFFFF : p, pmax = p;
  for (int o = 32; o > 0; o >>= 1) {
    pmin = min(pmin, __shfl_xor(pmin, o, 64));
    pmax = max(pmax, __shfl_xor(pmax, o, 64));
  }
  if (lane == 0) s_pmax[wave] = pmax;
  __syncthreads();
  pmax = max(max(s_pmax[0], s_pmax[1]), max(s_pmax[2], s_pmax[3]));
  const int n_tiles = (pmax + kMhKeys) / kMhKeys;           // tiles covering keys 0..pmax

  // ---- this lane's query as the B operand: dims 16ks + 8g .. +7 ----
  bf16x8 qf[kMhDqk / 16];
  {
    const int qr = qi < n_q ? qi : n_q - 1;
    const uint16_t* src = q + ((int64_t)qr * kHeads + h) * kMhDqk + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kMhDqk / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(src + 16 * ks);
  }

  // ---- tile staging: 32 keys of no-rope K, rope and V; 5 pieces of 16 B per thread ----
  u32x4 st[5];
  auto load_tile = [&](int t) {
    const int s0 = t * kMhKeys;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int pc = tid + kMhThreads * r;
      const int key = min(s0 + (pc >> 4), n_k - 1), c16 = pc & 15;
      st[r] = *reinterpret_cast<const u32x4*>(knope + ((int64_t)key * kHeads + h) * kMhDn + 8 * c16);
      st[3 + r] = *reinterpret_cast<const u32x4*>(vexp + ((int64_t)key * kHeads + h) * kMhDv + 8 * c16);
    }
    const int key = min(s0 + (tid >> 3), n_k - 1), c16 = tid & 7;
    st[2] = *reinterpret_cast<const u32x4*>(kv + (int64_t)key * kDqk + kDv + 8 * c16);
  };
  auto store_tile = [&](int buf) {
    uint8_t* sk = smem + buf * kMhBuf;
    uint8_t* sv = sk + kMhKBytes;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int pc = tid + kMhThreads * r;
      const int key = pc >> 4, c16 = pc & 15;
      *reinterpret_cast<u32x4*>(sk + key * kMhRowK + 16 * c16) = st[r];
      *reinterpret_cast<u32x4*>(sv + key * kMhRowV + 16 * c16) = st[3 + r];
    }
    *reinterpret_cast<u32x4*>(sk + (tid >> 3) * kMhRowK + 2 * kMhDn + 16 * (tid & 7)) = st[2];
  };

  f32x16 o[kMhDv / 32];
#pragma unroll
  for (int dt = 0; dt < kMhDv / 32; ++dt) o[dt] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  if (n_tiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const bool has_next = t + 1 < n_tiles;
    if (has_next) load_tile(t + 1);
    const uint8_t* sk = smem + buf * kMhBuf;
    const uint8_t* sv = sk + kMhKBytes;
    const int s0 = t * kMhKeys;

    // S^T = K . Q^T: rows are keys 8(i/4) + 4g + i%4, the lane's column its query
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kMhDqk / 16; ++ks) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(sk + col * kMhRowK + (16 * ks + 8 * g) * 2);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s, 0, 0, 0);
    }

    // online softmax per query column (log2 units)
    float z[16];
    if (s0 + kMhKeys - 1 <= pmin) {
#pragma unroll
      for (int i = 0; i < 16; ++i) z[i] = s[i] * scale_log2;
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = s0 + 8 * (i >> 2) + 4 * g + (i & 3);
        z[i] = key <= p ? s[i] * scale_log2 : -INFINITY;
      }
    }
    float tmax = z[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) tmax = fmaxf(tmax, z[i]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;   // no key yet: keep every weight 0
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    float psum = 0.f;
    bf16x8 pb[2];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = __builtin_amdgcn_exp2f(z[i] - m_use);
      psum += e;
      pb[i >> 3][i & 7] = (__bf16)e;
    }
    l_run = l_run * alpha + psum;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < kMhDv / 32; ++dt) o[dt] *= alpha;
    }
    m_run = m_new;

    // O^T += V^T . P^T: MFMA step j takes keys 16j + {4g..4g+3, 8+4g..8+4g+3}
    // in the lane group g, the order P holds them in; the transposed reads of
    // the 16-lane group G = lane >> 4 address key rows base + (lane & 15) >> 2
    // and columns 16(G & 1) + 4(lane & 3) .. +3, so lane l receives column
    // (l & 31) of the tile, four consecutive keys from base
    {
      const int jj = lane & 15, G = lane >> 4;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r0 = 16 * j + 4 * g + (jj >> 2);
#pragma unroll
        for (int dt = 0; dt < kMhDv / 32; ++dt) {
          const int cc = 32 * dt + 16 * (G & 1) + 4 * (jj & 3);
          const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((mh_lds_i16x4*)(sv + r0 * kMhRowV + 2 * cc));
          const i16x4 v1 =
              __builtin_amdgcn_ds_read_tr16_b64_v4i16((mh_lds_i16x4*)(sv + (r0 + 8) * kMhRowV + 2 * cc));
          const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[j], o[dt], 0, 0, 0);
        }
      }
    }
    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (qi >= n_q) return;
  // ---- normalise and write: the lane's query, dims 32dt + 8(i/4) + 4g + i%4 ----
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const int64_t o_row = ((int64_t)qi * kHeads + h) * kMhDv;
#pragma unroll
  for (int dt = 0; dt < kMhDv / 32; ++dt)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int d0 = 32 * dt + 8 * i4 + 4 * g;
      const f32x4 r = f32x4{o[dt][4 * i4], o[dt][4 * i4 + 1], o[dt][4 * i4 + 2], o[dt][4 * i4 + 3]} * inv;
      if constexpr (OUT_F32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(out) + o_row + d0) = r;
      } else {
        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + o_row + d0) =
            u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
      }
    }
  if (lse && g == 0)
    lse[(int64_t)qi * kHeads + h] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
}

size_t dense_mha_ws_bytes(int64_t n_k) { return (size_t)n_k * kHeads * (kMhDn + kMhDv) * 2; }

hipError_t launch_dense_mha(const DenseMhaArgs& A, hipStream_t st) {
  if (A.n_q <= 0) return hipSuccess;
  uint16_t* knope = static_cast<uint16_t*>(A.ws);
  uint16_t* vexp = knope + (size_t)A.n_k * kHeads * kMhDn;
  // the per-head keys and values: C_h[s][d] = sum_c kv[s][c] W[h][d][c]
  BmmArgs bk{A.kv, kDqk, 0, A.w_uk, kDv, (int64_t)kMhDn * kDv, false, knope, (int64_t)kHeads * kMhDn, kMhDn,
             (int)A.n_k, kMhDn, kDv, kHeads};
  hipError_t e = launch_bmm_bf16(bk, st);
  if (e != hipSuccess) return e;
  BmmArgs bv = bk;
  bv.B = A.w_uv;
  bv.C = vexp;
  e = launch_bmm_bf16(bv, st);
  if (e != hipSuccess) return e;
  const int n_qb = (A.n_q + kMhQ - 1) / kMhQ;
  const dim3 grid((unsigned)(n_qb * kHeads));
  const float scale_log2 = A.sm_scale * 1.4426950408889634f;
  if (A.out_f32)
    hipLaunchKernelGGL(dense_mha_kernel<true>, grid, dim3(kMhThreads), 0, st, A.q, A.kv, knope, vexp, A.q_pos, A.n_q,
                       (int)A.n_k, scale_log2, A.out, A.lse);
  else
    hipLaunchKernelGGL(dense_mha_kernel<false>, grid, dim3(kMhThreads), 0, st, A.q, A.kv, knope, vexp, A.q_pos,
                       A.n_q, (int)A.n_k, scale_log2, A.out, A.lse);
  return hipGetLastError();
}

}  // namespace sma
