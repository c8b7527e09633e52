// Per-query top-k selection over causal indexer scores (gfx950).
//
// Keeps the min(K, n) largest of a row's n scores, ties at the threshold to
// the lowest positions, written in ascending position order (the selection
// of 2,048 tokens per query in the GLM-5.3 part 2 article, "Pourquoi pas TP
// ou DP ?", with the tie-break reading).
//
// One 1024-thread workgroup per row, no atomics outside LDS, deterministic:
//  1. scores become order-preserving uint32 keys (-0.0 folded onto +0.0) and
//     the key range [lo, hi] of the row is found while they are loaded;
//  2. radix refinement: the range is cut into <= 2048 equal-width bins, an
//     LDS histogram locates the bin holding the K-th largest key, and the
//     range shrinks to that bin, until it is a single key T (at most three
//     11-bit rounds for 32-bit keys).  Because the bins span the row's
//     actual range rather than fixed bit fields, the first histogram is
//     spread over the scores' distribution and LDS atomics rarely collide.
//     After the first round the keys of the selected bin (normally a few
//     dozen) are copied to an LDS list and the later rounds run on that list
//     alone; a bin too full for the list is refined over the whole row;
//     When the bin holds at most 64 keys one wave ranks them directly;
//  3. an ordered compaction writes every position with key > T plus the
//     first (K - #greater) positions with key == T, each to the slot given by
//     a block-wide prefix count, so the output is ascending by position (for
//     rows held on chip each thread marks its positions in bit masks first).
// Rows up to 1024*V scores are read once into registers (blocked: thread t
// owns positions [t*V, t*V+V), so a wave whose positions all lie past the
// row end skips every pass); longer rows are streamed from memory in every
// full pass.
#include "sma_device.h"
#include "sma_launch.h"

namespace sma {

constexpr int kBins = 2048;
constexpr int kStreamV = 16;   // elements per thread per streamed chunk

template <int THREADS>
struct TopkShared {
  static constexpr int WAVES = THREADS / 64;
  uint32_t hist[kBins];
  uint32_t red[WAVES * 2];
  uint32_t bcast[4];
};

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive block-wide prefix of two counters at once (packed as 2 x 32 bit
// in a 64-bit lane value would overflow for long rows, so they are scanned
// separately through the same LDS slots).
template <int THREADS>
__device__ __forceinline__ void block_excl_scan2(uint32_t a, uint32_t b, uint32_t& ea, uint32_t& eb,
                                                 uint32_t& ta, uint32_t& tb, TopkShared<THREADS>& sh) {
  constexpr int kTopkWaves = THREADS / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t ia = wave_incl_scan(a, lane), ib = wave_incl_scan(b, lane);
  if (lane == 63) {
    sh.red[wave] = ia;
    sh.red[kTopkWaves + wave] = ib;
  }
  __syncthreads();
  uint32_t pa = 0, pb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const uint32_t xa = sh.red[w], xb = sh.red[kTopkWaves + w];
    if (w < wave) { pa += xa; pb += xb; }
    sa += xa;
    sb += xb;
  }
  ea = pa + ia - a;
  eb = pb + ib - b;
  ta = sa;
  tb = sb;
  __syncthreads();
}

template <int V>
struct RowSource {
  // V > 0: keys in registers; V == 0: streamed from `row`.
  uint32_t key[V > 0 ? V : 1];
};

template <int THREADS, int V, int VL>
__global__ __launch_bounds__(THREADS, 1) void topk_kernel(const float* __restrict__ scores,
                                                               int64_t ld,
                                                               const int32_t* __restrict__ q_pos,
                                                               int n_k, int K,
                                                               int32_t* __restrict__ idx) {
  constexpr int kTopkThreads = THREADS, kTopkWaves = THREADS / 64;
  static_assert(kBins % THREADS == 0, "whole histogram bins per thread");
  __shared__ TopkShared<THREADS> sh;
  // Keys of positions THREADS*V + tid*VL + j live in LDS at word j*THREADS + tid
  // (consecutive threads hit consecutive banks).
  __shared__ uint32_t lds_keys[VL > 0 ? VL * THREADS : 1];
  __shared__ uint32_t cand[kBins];   // keys of the selected bin after round 1
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;
  int p = q_pos[row];
  p = p < -1 ? -1 : (p > n_k - 1 ? n_k - 1 : p);
  const int n = p + 1;
  int32_t* out = idx + (int64_t)row * K;
  const float* src = scores + (int64_t)row * ld;

  if (n <= K) {
    for (int e = tid; e < K; e += kTopkThreads) out[e] = e < n ? e : -1;
    return;
  }

  // Positions past the row end carry key 0, below every real key (score_key
  // never returns 0), so no pass needs a per-position bound check.  A wave
  // whose positions of a segment all lie past the row end skips it.
  constexpr int kSeg2 = THREADS * V;   // first position held in LDS
  const bool act1 = V > 0 && wave * 64 * V < n;
  const bool act2 = VL > 0 && kSeg2 + wave * 64 * VL < n;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  auto note = [&](uint32_t k) {
    kmin = min(kmin, k ? k : 0xFFFFFFFFu);
    kmax = max(kmax, k);
  };
  RowSource<V> rs;
  if constexpr (V > 0) {
    if (act1) {
      const int base = tid * V;
#pragma unroll
      for (int v = 0; v < V; v += 4) {
        const int p0 = base + v;
        f32x4 x;
        if (p0 + 3 < n) {
          x = *reinterpret_cast<const f32x4*>(src + p0);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = p0 + e < n ? src[p0 + e] : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          rs.key[v + e] = p0 + e < n ? score_key(x[e]) : 0u;
          note(rs.key[v + e]);
        }
      }
    }
  }
  if constexpr (VL > 0) {
    if (act2) {
      const int base = kSeg2 + tid * VL;
#pragma unroll
      for (int v = 0; v < VL; v += 4) {
        const int p0 = base + v;
        f32x4 x;
        if (p0 + 3 < n) {
          x = *reinterpret_cast<const f32x4*>(src + p0);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = p0 + e < n ? src[p0 + e] : 0.f;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t k = p0 + e < n ? score_key(x[e]) : 0u;
          lds_keys[(v + e) * THREADS + tid] = k;
          note(k);
        }
      }
    }
  }

  // Visit every (position, key) of this thread; within each segment
  // (registers, then LDS) in ascending position.  Keys of positions >= n are 0.
  auto for_seg1 = [&](auto&& fn) {
    if (act1) {
      const int base = tid * V;
#pragma unroll
      for (int v = 0; v < V; ++v) fn(base + v, rs.key[v]);
    }
  };
  auto for_seg2 = [&](auto&& fn) {
    if (act2) {
      const int base = kSeg2 + tid * VL;
#pragma unroll 4
      for (int v = 0; v < VL; ++v) fn(base + v, lds_keys[v * THREADS + tid]);
    }
  };
  auto for_each = [&](auto&& fn) {
    if constexpr (V > 0) {
      for_seg1(fn);
      if constexpr (VL > 0) for_seg2(fn);
    } else {
      for (int c0 = 0; c0 < n; c0 += kTopkThreads * kStreamV) {
        const int base = c0 + tid * kStreamV;
#pragma unroll
        for (int v = 0; v < kStreamV; ++v) fn(base + v, base + v < n ? score_key(src[base + v]) : 0u);
      }
    }
  };

  // ---- 1. key range ----
  if constexpr (V == 0) for_each([&](int, uint32_t k) { note(k); });
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
  }
  if (lane == 0) {
    sh.red[wave] = kmin;
    sh.red[kTopkWaves + wave] = kmax;
  }
  __syncthreads();   // also publishes the LDS-resident keys
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    lo = min(lo, sh.red[w]);
    hi = max(hi, sh.red[kTopkWaves + w]);
  }
  __syncthreads();

  // ---- 2. radix refinement of [lo, hi] down to the threshold key ----
  uint32_t remaining = (uint32_t)K;   // still to take from keys inside [lo, hi]
  uint32_t in_range = 0;              // keys inside [lo, hi] after the last round
  auto refine = [&](auto&& visit) {
    const uint32_t width = hi - lo;
    const int bits = 32 - __clz(width);
    const int shift = bits > 11 ? bits - 11 : 0;
    const int nbins = (int)(width >> shift) + 1;
    for (int b = tid; b < nbins; b += kTopkThreads) sh.hist[b] = 0u;
    if (tid == 0) {
      sh.bcast[0] = 0u;
      sh.bcast[1] = 0u;
      sh.bcast[2] = 0u;
    }
    __syncthreads();
    visit([&](int, uint32_t k) {
      if (k >= lo && k <= hi) atomicAdd(&sh.hist[(k - lo) >> shift], 1u);
    });
    __syncthreads();
    // thread t owns bins [BPT*t, BPT*t + BPT); keys above a bin = total minus
    // the inclusive prefix up to and including it
    constexpr int BPT = kBins / THREADS;
    uint32_t hb[BPT], hsum = 0;
#pragma unroll
    for (int e = 0; e < BPT; ++e) {
      const int b = BPT * tid + e;
      hb[e] = b < nbins ? sh.hist[b] : 0u;
      hsum += hb[e];
    }
    uint32_t ex, dummy_e, tot, dummy_t;
    block_excl_scan2<THREADS>(hsum, 0u, ex, dummy_e, tot, dummy_t, sh);
    uint32_t above = tot - (ex + hsum);   // keys in bins past this thread's last bin
#pragma unroll
    for (int e = BPT - 1; e >= 0; --e) {
      const int b = BPT * tid + e;
      if (b < nbins && above < remaining && remaining <= above + hb[e]) {
        sh.bcast[0] = (uint32_t)b;
        sh.bcast[1] = above;
        sh.bcast[2] = hb[e];
      }
      above += hb[e];
    }
    __syncthreads();
    const uint32_t bsel = sh.bcast[0], above_sel = sh.bcast[1];
    in_range = sh.bcast[2];
    __syncthreads();
    remaining -= above_sel;
    const uint64_t nlo = (uint64_t)lo + ((uint64_t)bsel << shift);
    const uint64_t nhi = nlo + ((uint64_t)1 << shift) - 1;
    lo = (uint32_t)nlo;
    hi = (uint32_t)(nhi < (uint64_t)hi ? nhi : (uint64_t)hi);
  };
  // Each round shrinks the range by 11 bits: three rounds reach a single key;
  // the bound keeps the loops finite whatever the data.
  if (hi != lo) refine(for_each);
  if (hi != lo) {
    if (in_range <= (uint32_t)kBins) {
      if (tid == 0) sh.bcast[3] = 0u;
      __syncthreads();
      for_each([&](int, uint32_t k) {
        if (k >= lo && k <= hi) cand[atomicAdd(&sh.bcast[3], 1u)] = k;
      });
      __syncthreads();
      const int n_cand = (int)in_range;
      if (n_cand <= 64) {
        // One wave ranks the candidates against each other: T is the key
        // with fewer than `remaining` candidates above it and at least
        // `remaining` at or above it.
        if (wave == 0) {
          const uint32_t x = lane < n_cand ? cand[lane] : 0u;
          uint32_t gt = 0, ge = 0;
          for (int j = 0; j < n_cand; ++j) {
            const uint32_t y = (uint32_t)__shfl((int)x, j, 64);
            gt += y > x;
            ge += y >= x;
          }
          if (lane < n_cand && gt < remaining && remaining <= ge) {   // every such lane holds T
            sh.bcast[0] = x;
            sh.bcast[1] = remaining - gt;
          }
        }
        __syncthreads();
        lo = hi = sh.bcast[0];
        remaining = sh.bcast[1];
      } else {
        auto for_cand = [&](auto&& fn) {
          for (int c = tid; c < n_cand; c += kTopkThreads) fn(c, cand[c]);
        };
        for (int round = 1; round < 4 && hi != lo; ++round) refine(for_cand);
      }
    } else {
      for (int round = 1; round < 4 && hi != lo; ++round) refine(for_each);
    }
  }
  const uint32_t T = lo;
  const uint32_t need_ties = remaining;   // >= 1 keys equal to T are taken

  // ---- 3. ordered compaction ----
  if constexpr (V > 0) {
    // Per segment, a thread's positions are consecutive: one bit per
    // position marks key > T, another key == T.  The block-wide prefix of the
    // counts (packed: greater in the low 12 bits, at most K - 1 in total;
    // equal above them) gives each thread its first output slot.
    uint32_t mg1 = 0, me1 = 0, mg2 = 0, me2 = 0;
    for_seg1([&](int pos, uint32_t k) {
      const int b = pos - tid * V;
      mg1 |= (uint32_t)(k > T) << b;
      me1 |= (uint32_t)(k == T) << b;
    });
    if constexpr (VL > 0) {
      for_seg2([&](int pos, uint32_t k) {
        const int b = pos - (kSeg2 + tid * VL);
        mg2 |= (uint32_t)(k > T) << b;
        me2 |= (uint32_t)(k == T) << b;
      });
    }
    const uint32_t c1 = __popc(mg1) | ((uint32_t)__popc(me1) << 12);
    const uint32_t c2 = __popc(mg2) | ((uint32_t)__popc(me2) << 12);
    uint32_t b1, b2, t1, t2;
    block_excl_scan2<THREADS>(c1, c2, b1, b2, t1, t2, sh);
    auto emit = [&](uint32_t mg, uint32_t me, int base, uint32_t g_before, uint32_t e_before) {
      uint32_t m = mg | me;
      while (m) {
        const int b = __builtin_ctz(m);
        m &= m - 1;
        if ((mg >> b) & 1u) {
          const uint32_t slot = g_before + min(e_before, need_ties);
          if (slot < (uint32_t)K) out[slot] = base + b;
          ++g_before;
        } else {
          if (e_before < need_ties && g_before + e_before < (uint32_t)K) out[g_before + e_before] = base + b;
          ++e_before;
        }
      }
    };
    emit(mg1, me1, tid * V, b1 & 0xFFFu, b1 >> 12);
    if constexpr (VL > 0)
      emit(mg2, me2, kSeg2 + tid * VL, (t1 & 0xFFFu) + (b2 & 0xFFFu), (t1 >> 12) + (b2 >> 12));
  } else {
    uint32_t g_run = 0, e_run = 0;   // totals of earlier chunks
    for (int c0 = 0; c0 < n; c0 += kTopkThreads * kStreamV) {
      const int base = c0 + tid * kStreamV;
      uint32_t kk[kStreamV];
      uint32_t cg = 0, ce = 0;
#pragma unroll
      for (int v = 0; v < kStreamV; ++v) {
        kk[v] = base + v < n ? score_key(src[base + v]) : 0u;
        cg += kk[v] > T;
        ce += kk[v] == T;
      }
      uint32_t g_before, e_before, tg, te;
      block_excl_scan2<THREADS>(cg, ce, g_before, e_before, tg, te, sh);
      g_before += g_run;
      e_before += e_run;
#pragma unroll
      for (int v = 0; v < kStreamV; ++v) {
        const uint32_t k = kk[v];
        if (k > T) {
          const uint32_t slot = g_before + min(e_before, need_ties);
          if (slot < (uint32_t)K) out[slot] = base + v;
          ++g_before;
        } else if (k == T) {
          if (e_before < need_ties && g_before + e_before < (uint32_t)K) out[g_before + e_before] = base + v;
          ++e_before;
        }
      }
      g_run += tg;
      e_run += te;
    }
  }
}

// ---------------------------------------------------------------------------
// Rows of at most 4*THREADS*(S1+S2) positions, held on chip: thread t owns
// positions 4*THREADS*s + 4t + e (e < 4), steps s < S1 in registers and the
// next S2 steps in LDS, so every load reads 1 KiB per wave contiguously.
// The ordered output comes from two LDS bit maps over the row's positions
// (key > T, key == T) that the threads fill with atomic ORs; each thread then
// owns 64 consecutive positions of the maps.
// ---------------------------------------------------------------------------
template <int THREADS, int S1, int S2>
__global__ __launch_bounds__(THREADS, 1) void topk_chip_kernel(const float* __restrict__ scores, int64_t ld,
                                                               const int32_t* __restrict__ q_pos, int n_k,
                                                               int K, int32_t* __restrict__ idx) {
  constexpr int kWaves = THREADS / 64, kStep = 4 * THREADS;
  static_assert(kBins % THREADS == 0, "whole histogram bins per thread");
  static_assert(kStep * (S1 + S2) <= 32 * kBins, "bit maps cover the row");
  __shared__ TopkShared<THREADS> sh;
  __shared__ u32x4 lds_keys[S2 > 0 ? S2 * THREADS : 1];
  __shared__ uint32_t cand[kBins];   // keys of the selected bin; later the key > T bit map
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;
  int p = q_pos[row];
  p = p < -1 ? -1 : (p > n_k - 1 ? n_k - 1 : p);
  const int n = p + 1;
  int32_t* out = idx + (int64_t)row * K;
  const float* src = scores + (int64_t)row * ld;

  if (n <= K) {
    for (int e = tid; e < K; e += THREADS) out[e] = e < n ? e : -1;
    return;
  }

  // Positions past the row end carry key 0, below every real key (score_key
  // never returns 0).  A wave whose first position of a step lies past the
  // row end skips that step in every pass.
  auto active = [&](int s) { return kStep * s + 256 * wave < n; };
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  auto load4 = [&](int s) -> u32x4 {
    const int p0 = kStep * s + 4 * tid;
    f32x4 x;
    if (p0 + 3 < n) {
      x = *reinterpret_cast<const f32x4*>(src + p0);
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = p0 + e < n ? src[p0 + e] : 0.f;
    }
    u32x4 k;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      k[e] = p0 + e < n ? score_key(x[e]) : 0u;
      kmin = min(kmin, k[e] ? k[e] : 0xFFFFFFFFu);
      kmax = max(kmax, k[e]);
    }
    return k;
  };
  u32x4 rk[S1];
#pragma unroll
  for (int s = 0; s < S1; ++s)
    if (active(s)) rk[s] = load4(s);
#pragma unroll
  for (int s = 0; s < S2; ++s)
    if (active(S1 + s)) lds_keys[s * THREADS + tid] = load4(S1 + s);

  // Visit every (position, key) of this thread in ascending position.
  auto for_each = [&](auto&& fn) {
#pragma unroll
    for (int s = 0; s < S1; ++s)
      if (active(s)) {
#pragma unroll
        for (int e = 0; e < 4; ++e) fn(kStep * s + 4 * tid + e, rk[s][e]);
      }
#pragma unroll 2
    for (int s = 0; s < S2; ++s)
      if (active(S1 + s)) {
        const u32x4 k = lds_keys[s * THREADS + tid];
#pragma unroll
        for (int e = 0; e < 4; ++e) fn(kStep * (S1 + s) + 4 * tid + e, k[e]);
      }
  };

  // ---- 1. key range ----
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
  }
  if (lane == 0) {
    sh.red[wave] = kmin;
    sh.red[kWaves + wave] = kmax;
  }
  __syncthreads();   // also publishes the LDS-resident keys
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    lo = min(lo, sh.red[w]);
    hi = max(hi, sh.red[kWaves + w]);
  }
  __syncthreads();

  // ---- 2. threshold key T ----
  uint32_t remaining = (uint32_t)K, in_range = 0;
  auto refine = [&](auto&& visit) {
    const uint32_t width = hi - lo;
    const int bits = 32 - __clz(width);
    const int shift = bits > 11 ? bits - 11 : 0;
    const int nbins = (int)(width >> shift) + 1;
    for (int b = tid; b < nbins; b += THREADS) sh.hist[b] = 0u;
    if (tid == 0) sh.bcast[0] = sh.bcast[1] = sh.bcast[2] = 0u;
    __syncthreads();
    visit([&](int, uint32_t k) {
      if (k >= lo && k <= hi) atomicAdd(&sh.hist[(k - lo) >> shift], 1u);
    });
    __syncthreads();
    constexpr int BPT = kBins / THREADS;
    uint32_t hb[BPT], hsum = 0;
#pragma unroll
    for (int e = 0; e < BPT; ++e) {
      const int b = BPT * tid + e;
      hb[e] = b < nbins ? sh.hist[b] : 0u;
      hsum += hb[e];
    }
    uint32_t ex, dummy_e, tot, dummy_t;
    block_excl_scan2<THREADS>(hsum, 0u, ex, dummy_e, tot, dummy_t, sh);
    uint32_t above = tot - (ex + hsum);
#pragma unroll
    for (int e = BPT - 1; e >= 0; --e) {
      const int b = BPT * tid + e;
      if (b < nbins && above < remaining && remaining <= above + hb[e]) {
        sh.bcast[0] = (uint32_t)b;
        sh.bcast[1] = above;
        sh.bcast[2] = hb[e];
      }
      above += hb[e];
    }
    __syncthreads();
    const uint32_t bsel = sh.bcast[0], above_sel = sh.bcast[1];
    in_range = sh.bcast[2];
    __syncthreads();
    remaining -= above_sel;
    const uint64_t nlo = (uint64_t)lo + ((uint64_t)bsel << shift);
    const uint64_t nhi = nlo + ((uint64_t)1 << shift) - 1;
    lo = (uint32_t)nlo;
    hi = (uint32_t)(nhi < (uint64_t)hi ? nhi : (uint64_t)hi);
  };
  if (hi != lo) refine(for_each);
  if (hi != lo) {
    if (in_range <= (uint32_t)kBins) {
      if (tid == 0) sh.bcast[3] = 0u;
      __syncthreads();
      for_each([&](int, uint32_t k) {
        if (k >= lo && k <= hi) cand[atomicAdd(&sh.bcast[3], 1u)] = k;
      });
      __syncthreads();
      const int n_cand = (int)in_range;
      if (n_cand <= 64) {
        // One wave ranks the candidates against each other: T is the key
        // with fewer than `remaining` candidates above it and at least
        // `remaining` at or above it.
        if (wave == 0) {
          const uint32_t x = lane < n_cand ? cand[lane] : 0u;
          uint32_t gt = 0, ge = 0;
          for (int j = 0; j < n_cand; ++j) {
            const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)x, j);
            gt += y > x;
            ge += y >= x;
          }
          if (lane < n_cand && gt < remaining && remaining <= ge) {   // every such lane holds T
            sh.bcast[0] = x;
            sh.bcast[1] = remaining - gt;
          }
        }
        __syncthreads();
        lo = hi = sh.bcast[0];
        remaining = sh.bcast[1];
      } else {
        auto for_cand = [&](auto&& fn) {
          for (int c = tid; c < n_cand; c += THREADS) fn(c, cand[c]);
        };
        for (int round = 1; round < 4 && hi != lo; ++round) refine(for_cand);
      }
    } else {
      for (int round = 1; round < 4 && hi != lo; ++round) refine(for_each);
    }
  }
  const uint32_t T = lo;
  const uint32_t need_ties = remaining;   // >= 1 keys equal to T are taken

  // ---- 3. ordered compaction through two bit maps ----
  uint32_t* gmap = cand;      // key > T
  uint32_t* emap = sh.hist;   // key == T
  __syncthreads();            // every read of cand / hist is done
  for (int w = tid; w < kBins; w += THREADS) gmap[w] = emap[w] = 0u;
  __syncthreads();
  auto mark = [&](int s, const u32x4& k) {
    uint32_t g = 0, q = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      g |= (uint32_t)(k[e] > T) << e;
      q |= (uint32_t)(k[e] == T) << e;
    }
    const int word = (kStep * s + 4 * tid) >> 5, sh4 = 4 * (tid & 7);
    if (g) atomicOr(&gmap[word], g << sh4);
    if (q) atomicOr(&emap[word], q << sh4);
  };
#pragma unroll
  for (int s = 0; s < S1; ++s)
    if (active(s)) mark(s, rk[s]);
#pragma unroll 2
  for (int s = 0; s < S2; ++s)
    if (active(S1 + s)) mark(S1 + s, lds_keys[s * THREADS + tid]);
  __syncthreads();
  // thread t owns positions [64t, 64t + 64): map words 2t, 2t + 1
  uint32_t gw[2], ew[2];
  uint32_t cg = 0, ce = 0;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int w = 2 * tid + j;
    gw[j] = w < kBins ? gmap[w] : 0u;
    ew[j] = w < kBins ? emap[w] : 0u;
    cg += __popc(gw[j]);
    ce += __popc(ew[j]);
  }
  uint32_t g_before, e_before, tg, te;
  block_excl_scan2<THREADS>(cg, ce, g_before, e_before, tg, te, sh);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint32_t m = gw[j] | ew[j];
    while (m) {
      const int b = __builtin_ctz(m);
      m &= m - 1;
      const int pos = 64 * tid + 32 * j + b;
      if ((gw[j] >> b) & 1u) {
        const uint32_t slot = g_before + min(e_before, need_ties);
        if (slot < (uint32_t)K) out[slot] = pos;
        ++g_before;
      } else {
        if (e_before < need_ties && g_before + e_before < (uint32_t)K) out[g_before + e_before] = pos;
        ++e_before;
      }
    }
  }
}

bool topk_multi_wanted(int64_t n_k) { return n_k > 4 * 1024 * 16; }

hipError_t launch_topk(const TopkArgs& A, hipStream_t st) {
  if (A.n_q <= 0) return hipSuccess;
  if (topk_multi_wanted(A.n_k) && A.ws && A.ws_bytes >= topk_multi_bytes(A.n_q, A.n_k, A.top_k))
    return launch_topk_multi(A, A.ws, st);
  const dim3 grid((unsigned)A.n_q);
  // Rows that fit are read once and kept on chip: 1024 x 16 or 1024 x 32
  // keys in registers, or 1024 x 32 in registers plus 1024 x 32 in LDS (read
  // with 16-byte loads, so rows must start 16-byte aligned); longer or
  // unaligned rows are streamed from memory in every pass.
  const bool rows_aligned = (reinterpret_cast<uintptr_t>(A.scores) % 16 == 0) && (A.ld % 4 == 0);
  if (rows_aligned && A.n_k <= 4 * 1024 * 4) {
    hipLaunchKernelGGL((topk_chip_kernel<1024, 4, 0>), grid, dim3(1024), 0, st, A.scores, A.ld, A.q_pos,
                       (int)A.n_k, A.top_k, A.idx);
  } else if (rows_aligned && A.n_k <= 4 * 1024 * 8) {
    hipLaunchKernelGGL((topk_chip_kernel<1024, 8, 0>), grid, dim3(1024), 0, st, A.scores, A.ld, A.q_pos,
                       (int)A.n_k, A.top_k, A.idx);
  } else if (rows_aligned && A.n_k <= 4 * 1024 * 16) {
    hipLaunchKernelGGL((topk_chip_kernel<1024, 8, 8>), grid, dim3(1024), 0, st, A.scores, A.ld, A.q_pos,
                       (int)A.n_k, A.top_k, A.idx);
  } else {
    hipLaunchKernelGGL((topk_kernel<1024, 0, 0>), grid, dim3(1024), 0, st, A.scores, A.ld, A.q_pos,
                       (int)A.n_k, A.top_k, A.idx);
  }
  return hipGetLastError();
}

}  // namespace sma
