// Per-query top-k selection over causal indexer scores (gfx950).
//
// Keeps the min(K, n) largest of a row's n scores, ties at the threshold to
// the lowest positions, written in ascending position order (the selection
// of 2,048 tokens per query in the GLM-5.3 part 2 article, "Pourquoi pas TP
// ou DP ?", with the tie-break reading).
//
// Deterministic, no atomics outside LDS.  The exact selection, used on its
// own for long or unaligned rows (one 1024-thread workgroup per row, every
// pass streamed from memory):
//  1. scores become order-preserving uint32 keys (-0.0 folded onto +0.0) and
//     the key range [lo, hi] of the row is found;
//  2. radix refinement: the range is cut into <= 2048 equal-width bins, an
//     LDS histogram locates the bin holding the K-th largest key, and the
//     range shrinks to that bin, until it is a single key T (at most three
//     11-bit rounds for 32-bit keys).  Because the bins span the row's
//     actual range rather than fixed bit fields, the first histogram is
//     spread over the scores' distribution and LDS atomics rarely collide.
//     After the first round the keys of the selected bin (normally a few
//     dozen) are copied to an LDS list and the later rounds run on that list
//     alone; when it holds at most 64 keys one wave ranks them directly;
//  3. an ordered compaction writes every position with key > T plus the
//     first (K - #greater) positions with key == T, each to the slot given by
//     a block-wide prefix count, so the output is ascending by position.
// Aligned rows of at most 65,536 scores first keep only the positions at or
// above a threshold sampled from the row, in one pass, and run steps 2-3 on
// those (topk_filter_kernel below); rows longer than 65,536 scores, too few
// to fill the device one per workgroup, are split across workgroups when a
// workspace is given (topk_long_* below).
#include <type_traits>

#include "sma_device.h"
#include "sma_launch.h"

namespace sma {

constexpr int kBins = 2048;
// Elements per thread per streamed chunk.  The filtered kernel inlines the
// streaming selection as its fallback, so these arrays count towards its
// registers: at 8 the 16-bit-position kernel stays within four workgroups
// per CU (at 16 it needed three).
constexpr int kStreamV = 8;

// The score read for a position past a row's end: NaN.  score_or_nan (and
// the filter passes' quad_or_nan) select the address, never the load, so that
// the loads of a row's last, partial chunk are all in flight together
// instead of one round trip per guarded load.
__device__ __attribute__((aligned(16))) float g_past_row4[4] = {__builtin_nanf(""), __builtin_nanf(""),
                                                                 __builtin_nanf(""), __builtin_nanf("")};
__device__ __forceinline__ float score_or_nan(const float* src, int pos, int n) {
  return *(pos < n ? src + pos : g_past_row4);
}

// LDS scratch of a top-k workgroup: a BINS-bin histogram (BINS a power of
// two; a refinement round narrows a key range by log2(BINS) bits) and the
// block reductions' slots.
template <int THREADS, int BINS = kBins>
struct TopkShared {
  static constexpr int WAVES = THREADS / 64;
  static constexpr int kBinsN = BINS, kBinBits = __builtin_ctz(BINS);
  static_assert((BINS & (BINS - 1)) == 0, "a power-of-two bin count");
  alignas(16) uint32_t hist[BINS];
  uint32_t red[WAVES * 2];
  uint32_t bcast[4];
};

// Cross-lane steps by DPP (a VALU operand modifier) rather than by
// ds_bpermute, whose round trip through the LDS unit each step of a chain
// waits for.  dpp(v, CTRL, ROWS) reads v from the lane CTRL names; lanes with
// no such source, or outside the rows of the mask ROWS, read 0.
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xf, false);
}
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;   // lane 15 / 31 of a row into the next row(s)
constexpr int kDppQuadSwap1 = 0xB1, kDppQuadSwap2 = 0x4E;        // quad_perm [1,0,3,2] / [2,3,0,1]
constexpr int kDppHalfMirror = 0x141, kDppRowMirror = 0x140;     // mirror within 8 / 16 lanes

// Inclusive prefix sum over a wave: shifts by 1, 2, 4, 8 within each row of
// 16 lanes, then each row adds the total of the rows before it.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
  (void)lane;
  v += dpp<kDppRowShr1>(v);
  v += dpp<kDppRowShr2>(v);
  v += dpp<kDppRowShr4>(v);
  v += dpp<kDppRowShr8>(v);
  v += dpp<kDppRowBcast15, 0xa>(v);   // rows 1 and 3: + rows 0 and 2
  v += dpp<kDppRowBcast31, 0xc>(v);   // rows 2 and 3: + rows 0-1
  return v;
}

// Minimum and maximum over a wave, returned to every lane: butterflies
// within each row of 16 lanes, then the four rows' results read back.
__device__ __forceinline__ void wave_min_max(uint32_t& mn, uint32_t& mx) {
  mn = min(mn, dpp<kDppQuadSwap1>(mn));
  mx = max(mx, dpp<kDppQuadSwap1>(mx));
  mn = min(mn, dpp<kDppQuadSwap2>(mn));
  mx = max(mx, dpp<kDppQuadSwap2>(mx));
  mn = min(mn, dpp<kDppHalfMirror>(mn));
  mx = max(mx, dpp<kDppHalfMirror>(mx));
  mn = min(mn, dpp<kDppRowMirror>(mn));
  mx = max(mx, dpp<kDppRowMirror>(mx));
  mn = min(min((uint32_t)__builtin_amdgcn_readlane((int)mn, 0), (uint32_t)__builtin_amdgcn_readlane((int)mn, 16)),
           min((uint32_t)__builtin_amdgcn_readlane((int)mn, 32), (uint32_t)__builtin_amdgcn_readlane((int)mn, 48)));
  mx = max(max((uint32_t)__builtin_amdgcn_readlane((int)mx, 0), (uint32_t)__builtin_amdgcn_readlane((int)mx, 16)),
           max((uint32_t)__builtin_amdgcn_readlane((int)mx, 32), (uint32_t)__builtin_amdgcn_readlane((int)mx, 48)));
}

// Exclusive block-wide prefix of one counter, and its block total.
template <int THREADS, int BINS>
__device__ __forceinline__ void block_excl_scan(uint32_t a, uint32_t& ea, uint32_t& ta,
                                                TopkShared<THREADS, BINS>& sh) {
  constexpr int kTopkWaves = THREADS / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t ia = wave_incl_scan(a, lane);
  if (lane == 63) sh.red[wave] = ia;
  __syncthreads();
  uint32_t pa = 0, sa = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const uint32_t xa = sh.red[w];
    if (w < wave) pa += xa;
    sa += xa;
  }
  ea = pa + ia - a;
  ta = sa;
  __syncthreads();
}

// Exclusive block-wide prefix of two counters at once (packed as 2 x 32 bit
// in a 64-bit lane value would overflow for long rows, so they are scanned
// separately through the same LDS slots).
template <int THREADS, int BINS>
__device__ __forceinline__ void block_excl_scan2(uint32_t a, uint32_t b, uint32_t& ea, uint32_t& eb,
                                                 uint32_t& ta, uint32_t& tb, TopkShared<THREADS, BINS>& sh) {
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

// Exact top-k of one row streamed from memory in every pass (rows of any
// length, any alignment): key range, radix refinement to the threshold key
// T, ordered compaction.  Called by a whole THREADS-thread workgroup; `sh`
// and `cand` (BINS words) are its LDS scratch.
template <int THREADS, int BINS>
__device__ void topk_stream_row(const float* __restrict__ src, int n, int K, int32_t* __restrict__ out,
                                TopkShared<THREADS, BINS>& sh, uint32_t* cand) {
  constexpr int kTopkThreads = THREADS, kTopkWaves = THREADS / 64, kBits = TopkShared<THREADS, BINS>::kBinBits;
  static_assert(BINS % THREADS == 0, "whole histogram bins per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  auto note = [&](uint32_t k) {
    kmin = min(kmin, k ? k : 0xFFFFFFFFu);
    kmax = max(kmax, k);
  };
  // Visit every (position, key) of this thread; keys of positions >= n are 0
  // (below every real key: score_key never returns 0).
  auto for_each = [&](auto&& fn) {
    for (int c0 = 0; c0 < n; c0 += kTopkThreads * kStreamV) {
      const int base = c0 + tid * kStreamV;
      float x[kStreamV];
#pragma unroll
      for (int v = 0; v < kStreamV; ++v) x[v] = score_or_nan(src, base + v, n);
#pragma unroll
      for (int v = 0; v < kStreamV; ++v) fn(base + v, base + v < n ? score_key(x[v]) : 0u);
    }
  };

  // ---- 1. key range ----
  for_each([&](int, uint32_t k) { note(k); });
  wave_min_max(kmin, kmax);
  if (lane == 0) {
    sh.red[wave] = kmin;
    sh.red[kTopkWaves + wave] = kmax;
  }
  __syncthreads();
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
    const int shift = bits > kBits ? bits - kBits : 0;
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
    constexpr int BPT = BINS / THREADS;
    uint32_t hb[BPT], hsum = 0;
#pragma unroll
    for (int e = 0; e < BPT; ++e) {
      const int b = BPT * tid + e;
      hb[e] = b < nbins ? sh.hist[b] : 0u;
      hsum += hb[e];
    }
    uint32_t ex, tot;
    block_excl_scan<THREADS>(hsum, ex, tot, sh);
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
  // Each round shrinks the range by log2(BINS) >= 8 bits, so four rounds
  // reach a single key; the bound keeps the loops finite whatever the data.
  static_assert(4 * kBits >= 32, "four rounds narrow a 32-bit key range to one key");
  if (hi != lo) refine(for_each);
  if (hi != lo) {
    if (in_range <= (uint32_t)BINS) {
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
        __syncthreads();
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

  // ---- 3. ordered compaction: every position with key > T plus the first
  // need_ties positions with key == T, each to the slot a block-wide prefix
  // count gives it ----
  uint32_t g_run = 0, e_run = 0;   // totals of earlier chunks
  for (int c0 = 0; c0 < n; c0 += kTopkThreads * kStreamV) {
    const int base = c0 + tid * kStreamV;
    float x[kStreamV];
#pragma unroll
    for (int v = 0; v < kStreamV; ++v) x[v] = score_or_nan(src, base + v, n);
    uint32_t kk[kStreamV];
    uint32_t cg = 0, ce = 0;
#pragma unroll
    for (int v = 0; v < kStreamV; ++v) {
      kk[v] = base + v < n ? score_key(x[v]) : 0u;
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

// Rows of any length, one workgroup per row, every pass streamed.
template <int THREADS>
__global__ __launch_bounds__(THREADS, 1) void topk_stream_kernel(const float* __restrict__ scores, int64_t ld,
                                                                 const int32_t* __restrict__ q_pos, int n_k,
                                                                 int K, int32_t* __restrict__ idx) {
  __shared__ TopkShared<THREADS> sh;
  __shared__ uint32_t cand[kBins];
  const int row = blockIdx.x;
  int p = q_pos[row];
  p = p < -1 ? -1 : (p > n_k - 1 ? n_k - 1 : p);
  const int n = p + 1;
  int32_t* out = idx + (int64_t)row * K;
  if (n <= K) {
    for (int e = threadIdx.x; e < K; e += THREADS) out[e] = e < n ? e : -1;
    return;
  }
  topk_stream_row<THREADS>(scores + (int64_t)row * ld, n, K, out, sh, cand);
}

// ---------------------------------------------------------------------------
// Filtered top-k for 16-byte aligned rows (16-bit positions and four
// workgroups per CU up to 65,536 scores; 32-bit positions, a 4,096-score
// sample and three per CU beyond).  One 256-thread workgroup per row, one
// pass over the row:
//  1. a row longer than kFtCap takes a threshold from a sample of itself:
//     S/16 clusters of 16 consecutive scores spread evenly over the row (S =
//     2,048 or 4,096 samples).  One 2,048-bin histogram over the samples' key
//     range finds the bin holding the r0-th largest sample (a second one
//     within that bin when it holds more than kFtRefineBin samples, as with
//     scores of both signs, whose keys lie far apart); its lower edge is the
//     threshold, r0 chosen so that about 1.3 mu + 3 sqrt(mu) samples lie at
//     or above it (mu = K * S / n, the samples expected among the row's K
//     largest).  A shorter row keeps every key;
//  2. one coalesced pass keeps every position whose score is at or above the
//     threshold, with the score, in ascending position order: each wave owns
//     a contiguous quarter of an 8,192-score chunk, and wave ballots plus a
//     per-chunk table of the waves' counts give each kept position its LDS
//     slot (scores become keys only once kept);
//  3. if between K and kFtCap positions were kept, the threshold key T comes
//     from the kept keys alone (one histogram round, then one wave ranks the
//     few keys of the selected bin) and an ordered compaction over them
//     writes the row.  Every one of the K largest keys is at or above a
//     threshold that keeps K or more, so the result is exact; a row that kept
//     fewer than K or more than kFtCap is redone by the streaming selection
//     in the same workgroup.
// ---------------------------------------------------------------------------
constexpr int kFtThreads = 256;
constexpr int kFtWaves = kFtThreads / 64;
constexpr int kFtCap = 5120;                      // kept positions held in LDS (rows of > 32,768 scores)
// For rows of at most 32,768 scores the 16-bit-position kernel holds fewer
// (4,608) with a 1,024-bin histogram: 31 KiB of LDS, five workgroups per CU
// instead of four (such rows keep about 3,240 +- 300 with the 2,048-sample
// threshold).  Measured: the 16K top-k 0.29-0.36 -> 0.24-0.25 ms; with rows
// of up to 65,536 scores the fifth workgroup made it ~2.5% slower, so those
// keep four.
constexpr int kFtCap16 = 4608, kFtBins16 = 1024, kFtShortMax = 32768;
constexpr int kFtClusterLen = 16;                 // consecutive scores per sample cluster
constexpr int kFtU = 8;                           // 16-byte loads per thread per chunk
constexpr int kFtChunk = kFtThreads * 4 * kFtU;   // 8,192 positions
constexpr int kFtWaveSpan = 256 * kFtU;           // a wave's contiguous share of a chunk
constexpr int64_t kFtLongMax = 1 << 18;           // longest rows the filtered kernel takes
constexpr uint32_t kFtRefineBin = 32;             // samples in the threshold's bin that call for a second round

// Loads of a row's last, partial chunk.  On 16-byte aligned rows a lane
// whose four positions all lie inside the row loads them as one vector and
// a lane past the row's end loads four NaNs (which no threshold keeps) from
// g_past_row4: the address is selected, never the load, so the chunk's loads
// go out together instead of one round trip per guarded load.  The one lane
// that straddles the end (n not a multiple of 4) gets NaNs too; its n & 3
// in-row scores are read once per row (row_tail) and put back by fix_tail
// before the chunk is used.  Unaligned rows read each position through
// score_or_nan.
__device__ __forceinline__ f32x4 quad_or_nan(const float* src, int p0, int n) {   // p0 % 4 == 0
  return *reinterpret_cast<const f32x4*>(p0 + 3 < n ? src + p0 : g_past_row4);
}
struct RowTail {
  int n4;      // n & ~3: the straddling lane's first position
  float v[3];  // scores n4 .. n4 + 2 (those below n are used)
};
__device__ __forceinline__ RowTail row_tail(const float* src, int n) {   // n >= 1
  RowTail t;
  t.n4 = n & ~3;
#pragma unroll
  for (int e = 0; e < 3; ++e) t.v[e] = src[min(t.n4 + e, n - 1)];
  return t;
}
// pw: the lane's first position in the chunk; step u covers pw + 256u + 0..3.
__device__ __forceinline__ void fix_tail(f32x4 (&x)[kFtU], int pw, int n, const RowTail& t) {
#pragma unroll
  for (int u = 0; u < kFtU; ++u) {
    const int p0 = pw + 256 * u;
    if (p0 == t.n4 && p0 < n) {
#pragma unroll
      for (int e = 0; e < 3; ++e)
        if (p0 + e < n) x[u][e] = t.v[e];
    }
  }
}

// The score whose key is k (the inverse of score_key for finite scores).
__device__ __forceinline__ float key_score(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Range [lo, hi] of the nonzero keys the workgroup holds (the first m <= M
// registers per thread, m uniform; 0 = none).
template <int M, int BINS>
__device__ __forceinline__ void ft_range(const uint32_t (&key)[M], uint32_t& lo, uint32_t& hi,
                                         TopkShared<kFtThreads, BINS>& sh, int m = M) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    if (j < m) {
      kmin = min(kmin, key[j] ? key[j] : 0xFFFFFFFFu);
      kmax = max(kmax, key[j]);
    }
  }
  wave_min_max(kmin, kmax);
  if (lane == 0) {
    sh.red[wave] = kmin;
    sh.red[kFtWaves + wave] = kmax;
  }
  __syncthreads();
  lo = 0xFFFFFFFFu;
  hi = 0u;
#pragma unroll
  for (int w = 0; w < kFtWaves; ++w) {
    lo = min(lo, sh.red[w]);
    hi = max(hi, sh.red[kFtWaves + w]);
  }
  __syncthreads();
}

// One refinement round over the workgroup's keys (the first m <= M
// registers per thread, m uniform): cut [lo, hi] into <= BINS bins of equal
// width and keep the bin holding the remaining-th largest key at or above
// lo.  Keys above hi are counted in the last bin when open_top is set (its
// upper edge then becomes the largest key), and ignored otherwise.  Narrows
// lo, hi and remaining; returns how many keys the kept bin holds.  Thread 0
// also zeroes bcast[3] for a caller that gathers the bin's keys next.
template <int M, int BINS>
__device__ uint32_t ft_round(const uint32_t (&key)[M], uint32_t& lo, uint32_t& hi, uint32_t& remaining,
                             TopkShared<kFtThreads, BINS>& sh, int m = M, bool open_top = false) {
  constexpr int kBits = TopkShared<kFtThreads, BINS>::kBinBits;
  const int tid = threadIdx.x;
  const uint32_t width = hi - lo;
  const int bits = 32 - __clz(width);
  const int shift = bits > kBits ? bits - kBits : 0;
  const int nbins = (int)(width >> shift) + 1;
  for (int b = tid; b < nbins; b += kFtThreads) sh.hist[b] = 0u;
  if (tid == 0) sh.bcast[3] = 0u;
  __syncthreads();
  const uint32_t top = open_top ? 0xFFFFFFFFu : hi;
#pragma unroll
  for (int j = 0; j < M; ++j)
    if (j < m && key[j] >= lo && key[j] <= top) atomicAdd(&sh.hist[min((key[j] - lo) >> shift, (uint32_t)nbins - 1)], 1u);
  __syncthreads();
  constexpr int BPT = BINS / kFtThreads;
  uint32_t hb[BPT], hsum = 0;
#pragma unroll
  for (int e = 0; e < BPT; ++e) hb[e] = sh.hist[BPT * tid + e];   // all BINS words exist
#pragma unroll
  for (int e = 0; e < BPT; ++e) {
    hb[e] = BPT * tid + e < nbins ? hb[e] : 0u;
    hsum += hb[e];
  }
  uint32_t ex, tot;
  block_excl_scan<kFtThreads>(hsum, ex, tot, sh);
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
  // (no barrier after these reads: the next writer of bcast[0..2] is a later
  // round's, two barriers on, and the histogram's reads are all done)
  const uint32_t bsel = sh.bcast[0], above_sel = sh.bcast[1], in_bin = sh.bcast[2];
  remaining -= above_sel;
  const uint64_t nlo = (uint64_t)lo + ((uint64_t)bsel << shift);
  const uint64_t nhi = nlo + ((uint64_t)1 << shift) - 1;
  lo = (uint32_t)nlo;
  hi = open_top && (int)bsel == nbins - 1 ? 0xFFFFFFFFu : (uint32_t)(nhi < (uint64_t)hi ? nhi : (uint64_t)hi);
  return in_bin;
}

// Steps 3-4 of the filtered top-k: the K largest of C kept entries (K <= C
// <= KEEP * kFtThreads; raw score bits ckey[i] of ascending positions
// cpos[i], no NaN among them), written to out in ascending position order.
// Thread t holds entries M t .. M t + M - 1 (M = ceil(C / kFtThreads),
// made odd where that fits, so that the strided LDS reads fall on distinct
// banks) in registers from the start: the threshold rounds count them in
// any order, and the compaction takes each thread's run in list order after
// one block-wide scan of the runs' counts; loops over the registers stop at
// M.  The K selected positions are assembled in ckey (free once the keys are
// in registers) and written out in whole 16-byte pieces.  With klo > 0 every
// kept key is at least klo (the filter's threshold) and khi is an estimate of
// the largest (the sample's largest): the first round bins [klo, khi] with an
// open top instead of first reducing the keys' range.  Called by the whole
// kFtThreads-thread workgroup.
template <typename PosT, int KEEP, int BINS>
__device__ void ft_select_kept(uint32_t* ckey, const PosT* cpos, int C, int K, int32_t* __restrict__ out,
                               TopkShared<kFtThreads, BINS>& sh, uint32_t klo = 0u, uint32_t khi = 0u) {
  constexpr int kBits = TopkShared<kFtThreads, BINS>::kBinBits;
  const int tid = threadIdx.x, lane = tid & 63;
  int M = (C + kFtThreads - 1) / kFtThreads;
  if ((M & 1) == 0 && M < KEEP) ++M;
  M = __builtin_amdgcn_readfirstlane(M);
  const int e0 = M * tid;
  // ---- 3. exact threshold key T among the kept keys ----
  // (reads at clamped indices, all issued before any is used; entries past
  // the thread's run or the list get key 0, below every kept key)
  uint32_t kk[KEEP];
#pragma unroll
  for (int j = 0; j < KEEP; ++j) kk[j] = ckey[min(e0 + j, C - 1)];
#pragma unroll
  for (int j = 0; j < KEEP; ++j) kk[j] = j < M && e0 + j < C ? score_key(__uint_as_float(kk[j])) : 0u;
  uint32_t lo, hi, need_ties = (uint32_t)K;
  const bool bounded = klo != 0u && khi > klo;
  if (bounded) {
    lo = klo;
    hi = khi;
  } else {
    ft_range<KEEP>(kk, lo, hi, sh);
  }
  // A round narrows the range by kBits bits; the open-topped first round
  // may leave a range of up to 32 bits, hence one more round.
  for (int round = 0; round < (32 + kBits - 1) / kBits + 1 && hi != lo; ++round) {
    const uint32_t in_bin = ft_round<KEEP>(kk, lo, hi, need_ties, sh, KEEP, bounded && round == 0);
    if (hi != lo && in_bin <= 64) {
      // every wave ranks the bin's keys (gathered once): T has fewer than
      // need_ties of them above it and at least need_ties at or above it.
      // Each thread claims room for all of its bin keys with one atomic
      // (bcast[3] was zeroed by the round).
      uint32_t* list = sh.hist;
      uint32_t mine = 0;
#pragma unroll
      for (int j = 0; j < KEEP; ++j) mine += kk[j] >= lo && kk[j] <= hi;
      uint32_t at = mine ? atomicAdd(&sh.bcast[3], mine) : 0u;
#pragma unroll
      for (int j = 0; j < KEEP; ++j)
        if (kk[j] >= lo && kk[j] <= hi) list[at++] = kk[j];
      __syncthreads();
      const int nb = (int)in_bin;
      const uint32_t x = lane < nb ? list[lane] : 0u;
      uint32_t gt = 0, ge = 0;
      for (int j = 0; j < nb; ++j) {
        const uint32_t y = (uint32_t)__builtin_amdgcn_readlane((int)x, j);
        gt += y > x;
        ge += y >= x;
      }
      // every lane that qualifies holds T; take the first
      const uint64_t q = __ballot(lane < nb && gt < need_ties && need_ties <= ge);
      const int src = (int)__builtin_ctzll(q);
      const uint32_t Tk = (uint32_t)__builtin_amdgcn_readlane((int)x, src);
      need_ties -= (uint32_t)__builtin_amdgcn_readlane((int)gt, src);
      lo = hi = Tk;
    }
  }
  const uint32_t T = lo;

  // ---- 4. ordered compaction: every kept entry above T and the first
  // need_ties equal to T, in list (= position) order ----
  PosT pp[KEEP];
#pragma unroll
  for (int j = 0; j < KEEP; ++j) pp[j] = cpos[min(e0 + j, C - 1)];
  uint32_t cg = 0, ce = 0;
#pragma unroll
  for (int j = 0; j < KEEP; ++j) {
    cg += kk[j] > T;
    ce += kk[j] == T;
  }
  uint32_t g_run, e_run, tg, te;   // entries above / equal to T in earlier threads' runs
  block_excl_scan2<kFtThreads>(cg, ce, g_run, e_run, tg, te, sh);
  uint32_t* stage = ckey;
#pragma unroll
  for (int j = 0; j < KEEP; ++j) {
    const uint32_t k = kk[j];
    uint32_t slot = 0xFFFFFFFFu;
    if (k > T) slot = g_run + min(e_run, need_ties);
    if (k == T && e_run < need_ties) slot = g_run + e_run;
    g_run += k > T;
    e_run += k == T;
    if (slot < (uint32_t)K) stage[slot] = (uint32_t)pp[j];
  }
  __syncthreads();
  if ((K & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
    for (int i = 4 * tid; i < K; i += 4 * kFtThreads)
      *reinterpret_cast<u32x4*>(out + i) = *reinterpret_cast<const u32x4*>(&stage[i]);
  } else {
    for (int i = tid; i < K; i += kFtThreads) out[i] = (int32_t)stage[i];
  }
}

// PosT holds a position (uint16_t for rows of at most 65,536 scores); SPT
// samples per thread (SPT * 256 in all); CAP kept positions in LDS; BINS
// histogram bins.
template <typename PosT, int SPT, int OCC, int CAP, int BINS>
__global__ __launch_bounds__(kFtThreads, OCC) void topk_filter_kernel(const float* __restrict__ scores, int64_t ld,
                                                                      const int32_t* __restrict__ q_pos, int n_k,
                                                                      int K, int32_t* __restrict__ idx) {
  constexpr int kSamples = kFtThreads * SPT, kClusters = kSamples / kFtClusterLen;
  static_assert(SPT % 4 == 0 && kFtClusterLen % SPT == 0, "whole 16-byte loads within one cluster");
  static_assert(CAP % kFtThreads == 0 && CAP + 4 >= BINS, "whole kept keys per thread; room for the fallback");
  __shared__ TopkShared<kFtThreads, BINS> sh;
  __shared__ alignas(16) uint32_t ckey[CAP + 4];   // score bits of the kept positions (the streaming fallback's scratch)
  __shared__ PosT cpos[CAP + 4];       // kept positions, ascending
  __shared__ uint32_t tab[2][kFtWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Later rows of a causal batch are the longer ones: hand them out first,
  // so that the last workgroups to start are short (64K: ~1%).  Keeping
  // neighbouring rows together matters more: interleaving short and long
  // rows across the launch was 30% slower.
  const int row = (int)gridDim.x - 1 - (int)blockIdx.x;
  int p = q_pos[row];
  p = p < -1 ? -1 : (p > n_k - 1 ? n_k - 1 : p);
  const int n = p + 1;
  int32_t* out = idx + (int64_t)row * K;
  const float* src = scores + (int64_t)row * ld;
  if (n <= K) {
    for (int e = tid; e < K; e += kFtThreads) out[e] = e < n ? e : -1;
    return;
  }

  // Wave w's step u of the chunk at c0 covers positions c0 + 2048w + 256u ..
  // + 255, lane l the four at + 4l; positions at or past n read as NaN, which
  // no threshold keeps.
  auto load = [&](int c0, f32x4 (&x)[kFtU]) {
    const int pw = c0 + kFtWaveSpan * wave + 4 * lane;
    if (c0 + kFtChunk <= n) {
#pragma unroll
      for (int u = 0; u < kFtU; ++u) x[u] = *reinterpret_cast<const f32x4*>(src + pw + 256 * u);
    } else {
#pragma unroll
      for (int u = 0; u < kFtU; ++u) x[u] = quad_or_nan(src, pw + 256 * u, n);
    }
  };
  const RowTail tail = row_tail(src, n);

  // ---- 1. threshold (the sample loads go out with the first chunk's) ----
  f32x4 sv[SPT / 4] = {};
  const bool sampled = n > CAP;
  if (sampled) {   // thread t loads SPT consecutive scores of cluster t*SPT/16
    const int c = tid * SPT / kFtClusterLen;
    const int start = (int)(((int64_t)c * (n - kFtClusterLen)) / (kClusters - 1)) & ~3;
#pragma unroll
    for (int v = 0; v < SPT / 4; ++v)
      sv[v] = *reinterpret_cast<const f32x4*>(src + start + (tid * SPT) % kFtClusterLen + 4 * v);
  }
  f32x4 xa[kFtU], xb[kFtU];
  load(0, xa);
  float thr = -INFINITY;
  uint32_t klo = 0u, khi = 0u;   // the threshold's key and the largest sample's (0: no sample)
  if (sampled) {
    uint32_t sk[SPT];
#pragma unroll
    for (int v = 0; v < SPT; ++v) sk[v] = score_key(sv[v >> 2][v & 3]);
    const float mu = (float)K * (float)kSamples / (float)n;
    const uint32_t r0 = (uint32_t)fminf(ceilf(1.3f * mu + 3.f * sqrtf(mu) + 4.f), (float)kSamples);
    uint32_t lo, hi, rem = r0;
    ft_range<SPT>(sk, lo, hi, sh);
    khi = __builtin_amdgcn_readfirstlane(hi);   // uniform: kept in a scalar register across the pass
    if (hi != lo) {
      // a key range spanning both signs leaves coarse bins near the top:
      // one more round when the kept bin holds many samples
      const uint32_t in_bin = ft_round<SPT>(sk, lo, hi, rem, sh);
      if (hi != lo && in_bin > kFtRefineBin) ft_round<SPT>(sk, lo, hi, rem, sh);
    }
    thr = key_score(lo);   // at least r0 samples lie at or above it
    klo = __builtin_amdgcn_readfirstlane(lo);
  }

  // ---- 2. one pass: positions with score >= thr, in ascending order ----
  uint32_t kept = 0;   // positions kept by earlier chunks
  // Keep the chunk at c0 (held in x), then load the chunk two ahead into x.
  // The kept list holds raw score bits; keys are formed for kept entries only.
  auto step = [&](int c0, int ci, f32x4 (&x)[kFtU]) {
    if (c0 + kFtChunk > n) fix_tail(x, c0 + kFtWaveSpan * wave + 4 * lane, n, tail);
    // off[u]: this lane's first slot for step u within the wave's kept
    // entries of the chunk (ballot prefix counts, accumulated by mbcnt)
    uint32_t off[kFtU];
    uint32_t wcnt = 0;
#pragma unroll
    for (int u = 0; u < kFtU; ++u) {
      uint32_t o = wcnt;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint64_t m = __ballot(x[u][e] >= thr);
        o = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, o));
        wcnt += (uint32_t)__popcll(m);
      }
      asm volatile("" : "+v"(o));   // keep the offset in a register (not recomputed after the barrier)
      off[u] = o;
    }
    if (lane == 0) tab[ci & 1][wave] = wcnt;
    __syncthreads();
    uint32_t base = kept, all = 0;
#pragma unroll
    for (int w = 0; w < kFtWaves; ++w) {
      const uint32_t v = tab[ci & 1][w];
      base += w < wave ? v : 0u;
      all += v;
    }
    const int pw = c0 + kFtWaveSpan * wave + 4 * lane;
    // a position not kept writes to this thread's own words of the
    // histogram, idle during this pass, so that no lane branches
#pragma unroll
    for (int u = 0; u < kFtU; ++u) {
      uint32_t slot = min(base + off[u], (uint32_t)CAP);   // slots CAP.. absorb an overflow
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const bool f = x[u][e] >= thr;
        uint32_t* kp = f ? &ckey[slot] : &sh.hist[tid];
        PosT* pp = f ? &cpos[slot] : reinterpret_cast<PosT*>(&sh.hist[kFtThreads + tid]);
        *pp = (PosT)(pw + 256 * u + e);
        *kp = __float_as_uint(x[u][e]);
        slot += f;
      }
    }
    kept += all;
    if (c0 + 2 * kFtChunk < n) load(c0 + 2 * kFtChunk, x);
  };
  if (kFtChunk < n) load(kFtChunk, xb);
  for (int c0 = 0, ci = 0; c0 < n; c0 += 2 * kFtChunk, ci += 2) {
    step(c0, ci, xa);
    if (c0 + kFtChunk < n) step(c0 + kFtChunk, ci + 1, xb);
  }
  __syncthreads();   // kept positions and keys are visible

  if (kept < (uint32_t)K || kept > (uint32_t)CAP) {   // threshold too high, or too many kept
    topk_stream_row<kFtThreads>(src, n, K, out, sh, ckey);
    return;
  }

  ft_select_kept<PosT, CAP / kFtThreads>(ckey, cpos, (int)kept, K, out, sh, klo, khi);
}

// ---------------------------------------------------------------------------
// Long rows split across workgroups: rows of more than 65,536 scores when
// there are too few of them to fill the device with one workgroup per row
// (a decode batch of 64 rows of ~1M scores).  One pass over each row:
//  1. topk_long_sample: one workgroup per row takes the filtered kernel's
//     threshold (step 1 above) from kLgSamples samples, 1,024 clusters of 16
//     consecutive scores spread evenly over the row, and stores it;
//  2. topk_long_filter: one workgroup per kLgChunk-score chunk of a row keeps,
//     as step 2 does, every position whose score is at or above the row's
//     threshold, in ascending order, into the chunk's list in the workspace
//     ((position, score bits); the first kLgChunkCap) with its count;
//  3. topk_long_final: one workgroup per row concatenates its chunks' lists
//     in chunk order and runs steps 3-4 on them.  A row that kept fewer than
//     K or more than kLgCap, or a chunk more than kLgChunkCap, is redone by
//     the streaming selection in that workgroup, so the result is exact.
// With 16,384 samples a row of 1M scores keeps about 4,000 +- 500 (K =
// 2,048); a row of at most kLgCap scores keeps all of them.
// ---------------------------------------------------------------------------
constexpr int kLgChunk = 2 * kFtChunk;                 // 16,384 positions per chunk workgroup
constexpr int kLgClusters = 1024;
constexpr int kLgSamples = kLgClusters * kFtClusterLen;   // 16,384
constexpr int kLgSPT = kLgSamples / kFtThreads;          // 64: four clusters per thread
constexpr int kLgCap = 8192;                           // kept entries a row's final workgroup holds
constexpr int kLgKeep = kLgCap / kFtThreads;            // 32 per thread
constexpr int kLgChunkCap = 4096;                      // kept entries a chunk's list holds

__device__ __forceinline__ int lg_row_len(const int32_t* q_pos, int row, int n_k) {
  int p = q_pos[row];
  p = p < -1 ? -1 : (p > n_k - 1 ? n_k - 1 : p);
  return p + 1;
}

template <bool ALIGNED>
__global__ __launch_bounds__(kFtThreads) void topk_long_sample(const float* __restrict__ scores, int64_t ld,
                                                               const int32_t* __restrict__ q_pos, int n_k, int K,
                                                               float* __restrict__ thr) {
  __shared__ TopkShared<kFtThreads> sh;
  const int row = blockIdx.x, tid = threadIdx.x;
  const int n = lg_row_len(q_pos, row, n_k);
  if (n <= kLgCap) {   // keeps every score (a row of at most K scores takes them all in step 3)
    if (tid == 0) thr[row] = -INFINITY;
    return;
  }
  const float* src = scores + (int64_t)row * ld;
  uint32_t sk[kLgSPT];
#pragma unroll
  for (int q = 0; q < kLgSPT / kFtClusterLen; ++q) {
    const int c = tid * (kLgSPT / kFtClusterLen) + q;
    const int start = (int)(((int64_t)c * (n - kFtClusterLen)) / (kLgClusters - 1)) & ~3;
#pragma unroll
    for (int v = 0; v < kFtClusterLen / 4; ++v) {
      f32x4 x;
      if constexpr (ALIGNED) {
        x = *reinterpret_cast<const f32x4*>(src + start + 4 * v);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = src[start + 4 * v + e];
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sk[kFtClusterLen * q + 4 * v + e] = score_key(x[e]);
    }
  }
  const float mu = (float)K * (float)kLgSamples / (float)n;
  const uint32_t r0 = (uint32_t)fminf(ceilf(1.3f * mu + 3.f * sqrtf(mu) + 4.f), (float)kLgSamples);
  uint32_t lo, hi, rem = r0;
  ft_range<kLgSPT>(sk, lo, hi, sh);
  if (hi != lo) {
    const uint32_t in_bin = ft_round<kLgSPT>(sk, lo, hi, rem, sh);
    if (hi != lo && in_bin > kFtRefineBin) ft_round<kLgSPT>(sk, lo, hi, rem, sh);
  }
  if (tid == 0) thr[row] = key_score(lo);   // at least r0 samples lie at or above it
}

template <bool ALIGNED>
__global__ __launch_bounds__(kFtThreads) void topk_long_filter(const float* __restrict__ scores, int64_t ld,
                                                               const int32_t* __restrict__ q_pos, int n_k, int K,
                                                               const float* __restrict__ thr, int nch,
                                                               uint2* __restrict__ list, uint32_t* __restrict__ cnt) {
  __shared__ uint32_t tab[2][kFtWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.y, chunk = blockIdx.x;
  const int n = lg_row_len(q_pos, row, n_k);
  const int64_t slot0 = (int64_t)row * nch + chunk;
  const int cbeg = chunk * kLgChunk;
  if (n <= K || cbeg >= n) {
    if (tid == 0) cnt[slot0] = 0u;
    return;
  }
  const float t = thr[row];
  const float* src = scores + (int64_t)row * ld;
  uint2* my = list + slot0 * kLgChunkCap;
  // Wave w's step u of the 8,192-position half at c0 covers c0 + 2048w +
  // 256u .. + 255, lane l the four at + 4l; positions at or past n read as
  // NaN, which no threshold keeps.
  auto load = [&](int c0, f32x4 (&x)[kFtU]) {
    const int pw = c0 + kFtWaveSpan * wave + 4 * lane;
    if (!ALIGNED) {
#pragma unroll
      for (int u = 0; u < kFtU; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) x[u][e] = score_or_nan(src, pw + 256 * u + e, n);
    } else if (c0 + kFtChunk <= n) {
#pragma unroll
      for (int u = 0; u < kFtU; ++u) x[u] = *reinterpret_cast<const f32x4*>(src + pw + 256 * u);
    } else {
#pragma unroll
      for (int u = 0; u < kFtU; ++u) x[u] = quad_or_nan(src, pw + 256 * u, n);
    }
  };
  f32x4 xa[kFtU], xb[kFtU];
  load(cbeg, xa);
  if (cbeg + kFtChunk < n) load(cbeg + kFtChunk, xb);
  RowTail tail{};
  if (ALIGNED && cbeg + 2 * kFtChunk > n) tail = row_tail(src, n);   // this workgroup holds the row's end
  uint32_t kept = 0;
  auto step = [&](int c0, int ci, f32x4 (&x)[kFtU]) {
    if (ALIGNED && c0 + kFtChunk > n) fix_tail(x, c0 + kFtWaveSpan * wave + 4 * lane, n, tail);
    uint32_t off[kFtU];
    uint32_t wcnt = 0;
#pragma unroll
    for (int u = 0; u < kFtU; ++u) {
      uint32_t o = wcnt;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint64_t m = __ballot(x[u][e] >= t);
        o = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, o));
        wcnt += (uint32_t)__popcll(m);
      }
      off[u] = o;
    }
    if (lane == 0) tab[ci][wave] = wcnt;
    __syncthreads();
    uint32_t base = kept, all = 0;
#pragma unroll
    for (int w = 0; w < kFtWaves; ++w) {
      const uint32_t v = tab[ci][w];
      base += w < wave ? v : 0u;
      all += v;
    }
    const int pw = c0 + kFtWaveSpan * wave + 4 * lane;
#pragma unroll
    for (int u = 0; u < kFtU; ++u) {
      uint32_t slot = base + off[u];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (x[u][e] >= t) {
          if (slot < (uint32_t)kLgChunkCap) my[slot] = make_uint2((uint32_t)(pw + 256 * u + e), __float_as_uint(x[u][e]));
          ++slot;
        }
      }
    }
    kept += all;
  };
  step(cbeg, 0, xa);
  if (cbeg + kFtChunk < n) step(cbeg + kFtChunk, 1, xb);
  if (tid == 0) cnt[slot0] = kept;
}

__global__ __launch_bounds__(kFtThreads) void topk_long_final(const float* __restrict__ scores, int64_t ld,
                                                              const int32_t* __restrict__ q_pos, int n_k, int K,
                                                              int nch, const uint2* __restrict__ list,
                                                              const uint32_t* __restrict__ cnt,
                                                              int32_t* __restrict__ idx) {
  __shared__ TopkShared<kFtThreads> sh;
  __shared__ alignas(16) uint32_t ckey[kLgCap];   // kept score bits (the streaming fallback's scratch)
  __shared__ int32_t cpos[kLgCap];    // kept positions, ascending
  __shared__ uint32_t s_off[kFtThreads];
  __shared__ uint32_t s_fail;
  const int row = blockIdx.x, tid = threadIdx.x;
  const int n = lg_row_len(q_pos, row, n_k);
  int32_t* out = idx + (int64_t)row * K;
  const float* src = scores + (int64_t)row * ld;
  if (n <= K) {
    for (int e = tid; e < K; e += kFtThreads) out[e] = e < n ? e : -1;
    return;
  }
  const int nc = (n + kLgChunk - 1) / kLgChunk;
  const uint32_t* rc = cnt + (int64_t)row * nch;
  const uint2* rl = list + (int64_t)row * nch * kLgChunkCap;
  if (tid == 0) s_fail = 0u;
  __syncthreads();
  // Concatenate the chunks' lists, kFtThreads chunks at a time: their counts
  // are scanned first, then entry g of the group lies in the last chunk whose
  // offset is <= g (an empty chunk shares its offset with the next one).
  uint32_t total = 0;
  for (int g0 = 0; g0 < nc; g0 += kFtThreads) {
    const int c = g0 + tid;
    const uint32_t v = c < nc ? rc[c] : 0u;
    if (v > (uint32_t)kLgChunkCap) s_fail = 1u;
    uint32_t ex, tv;
    block_excl_scan<kFtThreads>(v, ex, tv, sh);
    s_off[tid] = total + ex;
    __syncthreads();
    if (s_fail || total + tv > (uint32_t)kLgCap) {
      total += tv;
      break;
    }
    const int gn = min(kFtThreads, nc - g0);
    for (uint32_t g = total + tid; g < total + tv; g += kFtThreads) {
      int lo = 0, hi = gn - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_off[mid] <= g) lo = mid;
        else hi = mid - 1;
      }
      const uint2 e = rl[(int64_t)(g0 + lo) * kLgChunkCap + (g - s_off[lo])];
      cpos[g] = (int32_t)e.x;
      ckey[g] = e.y;
    }
    total += tv;
    __syncthreads();
  }
  __syncthreads();
  if (s_fail || total < (uint32_t)K || total > (uint32_t)kLgCap) {   // threshold too high, or too many kept
    topk_stream_row<kFtThreads>(src, n, K, out, sh, ckey);
    return;
  }
  ft_select_kept<int32_t, kLgKeep>(ckey, cpos, (int)total, K, out, sh);
}

bool topk_long_wanted(int64_t n_k) { return n_k > 65536; }

size_t topk_long_bytes(int32_t n_q, int64_t n_k, int32_t top_k) {
  (void)top_k;
  if (n_q <= 0 || n_k <= 0) return 0;
  const int64_t nch = (n_k + kLgChunk - 1) / kLgChunk;
  auto al = [](size_t b) { return (b + 255) / 256 * 256; };
  return al((size_t)n_q * 4) + al((size_t)n_q * nch * 4) + al((size_t)n_q * nch * kLgChunkCap * 8);
}

static hipError_t launch_topk_long(const TopkArgs& A, bool aligned, hipStream_t st) {
  const int nch = (int)((A.n_k + kLgChunk - 1) / kLgChunk);
  auto al = [](size_t b) { return (b + 255) / 256 * 256; };
  uint8_t* p = static_cast<uint8_t*>(A.ws);
  float* thr = reinterpret_cast<float*>(p);
  p += al((size_t)A.n_q * 4);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(p);
  p += al((size_t)A.n_q * nch * 4);
  uint2* list = reinterpret_cast<uint2*>(p);
  const dim3 rows((unsigned)A.n_q), chunks((unsigned)nch, (unsigned)A.n_q);
  if (aligned) {
    hipLaunchKernelGGL(topk_long_sample<true>, rows, dim3(kFtThreads), 0, st, A.scores, A.ld, A.q_pos, (int)A.n_k,
                       A.top_k, thr);
    hipLaunchKernelGGL(topk_long_filter<true>, chunks, dim3(kFtThreads), 0, st, A.scores, A.ld, A.q_pos,
                       (int)A.n_k, A.top_k, thr, nch, list, cnt);
  } else {
    hipLaunchKernelGGL(topk_long_sample<false>, rows, dim3(kFtThreads), 0, st, A.scores, A.ld, A.q_pos,
                       (int)A.n_k, A.top_k, thr);
    hipLaunchKernelGGL(topk_long_filter<false>, chunks, dim3(kFtThreads), 0, st, A.scores, A.ld, A.q_pos,
                       (int)A.n_k, A.top_k, thr, nch, list, cnt);
  }
  hipLaunchKernelGGL(topk_long_final, rows, dim3(kFtThreads), 0, st, A.scores, A.ld, A.q_pos, (int)A.n_k, A.top_k,
                     nch, list, cnt, A.idx);
  return hipGetLastError();
}



hipError_t launch_topk(const TopkArgs& A, hipStream_t st) {
  if (A.n_q <= 0) return hipSuccess;
  const bool rows_aligned = (reinterpret_cast<uintptr_t>(A.scores) % 16 == 0) && (A.ld % 4 == 0);
  const dim3 grid((unsigned)A.n_q);
  // Long rows with enough of them to fill the device (a few workgroups per
  // CU) take the filtered kernel too, with 32-bit positions, up to the row
  // length whose expected kept count stays well inside the LDS slots: the
  // 4,096-sample threshold keeps about 1.3K + 3 sqrt(K n / 4096) + n / 1024
  // scores of an n-score row (about 4,000 +- 510 at n = 2^18 with K = 2,048,
  // 4,710 +- 780 at 2^19, against kFtCap = 5,120 slots); a row that
  // overflows is redone by the streaming selection, several passes over it.
  if (rows_aligned && A.n_k > 65536 && A.n_k <= kFtLongMax && A.n_q >= 4 * device_cu_count()) {
    hipLaunchKernelGGL((topk_filter_kernel<uint32_t, 16, 3, kFtCap, kBins>), grid, dim3(kFtThreads), 0, st,
                       A.scores, A.ld, A.q_pos, (int)A.n_k, A.top_k, A.idx);
    return hipGetLastError();
  }
  if (topk_long_wanted(A.n_k) && A.ws && A.ws_bytes >= topk_long_bytes(A.n_q, A.n_k, A.top_k))
    return launch_topk_long(A, rows_aligned, st);
  // 16-byte aligned rows of up to 65,536 scores take the filtered kernel
  // (one pass over the row); longer or unaligned rows are streamed from
  // memory in every pass.
  if (rows_aligned && A.n_k <= kFtShortMax) {
    hipLaunchKernelGGL((topk_filter_kernel<uint16_t, 8, 5, kFtCap16, kFtBins16>), grid, dim3(kFtThreads), 0, st,
                       A.scores, A.ld, A.q_pos, (int)A.n_k, A.top_k, A.idx);
  } else if (rows_aligned && A.n_k <= 65536) {
    hipLaunchKernelGGL((topk_filter_kernel<uint16_t, 8, 4, kFtCap, kBins>), grid, dim3(kFtThreads), 0, st,
                       A.scores, A.ld, A.q_pos, (int)A.n_k, A.top_k, A.idx);
  } else {
    hipLaunchKernelGGL((topk_stream_kernel<1024>), grid, dim3(1024), 0, st, A.scores, A.ld, A.q_pos,
                       (int)A.n_k, A.top_k, A.idx);
  }
  return hipGetLastError();
}

}  // namespace sma
