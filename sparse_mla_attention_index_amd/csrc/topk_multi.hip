// Top-k over long score rows, split across workgroups (gfx950).
//
// Same selection as topk.hip (the 2,048 best earlier tokens of each query,
// GLM-5.3 part 2, "Pourquoi pas TP ou DP ?"; ties at the threshold to the
// lowest positions; ascending output), for rows too long to hold on chip or
// too few to fill the GPU (a PCP rank's 128K-token rows, a decode batch of
// 64 rows of ~1M scores).  Each row is cut into chunks of kChunk scores and
// every chunk is a workgroup, so all CUs stream:
//   1. tkm_minmax  - per-row key range [lo, hi] (integer atomics);
//   2. three rounds of tkm_hist + tkm_select - a 2,048-bin histogram of the
//      keys inside [lo, hi] (bins follow the row's own range, so the first
//      round already isolates the threshold to ~n/2048 keys), then the bin
//      holding the K-th largest key becomes the new [lo, hi]; a row stops
//      refining once at most K keys remain inside or the range is one key;
//   3. tkm_collect - one more pass writes, per chunk and in position order,
//      the positions above hi (all selected) and the (position, key) pairs
//      inside [lo, hi] (candidates; at most K per chunk are kept, enough
//      because at most K are ever taken);
//   4. tkm_final   - per row: picks the candidates (the best `rem` by key,
//      ties to the lowest positions) and merges them with the positions
//      above hi into the ascending output.
// All counts are integers and every list is built in position order, so the
// result is deterministic.  Work buffers live in the caller's workspace.
#include "sma_device.h"
#include "sma_launch.h"

namespace sma {
namespace {

constexpr int kChunk = 16384;       // scores per chunk workgroup
constexpr int kTkmThreads = 512;    // threads of the chunk workgroups
constexpr int kTkmBins = 2048;
constexpr int kFinalThreads = 1024;

struct RowState {
  uint32_t lo, hi;    // key range still being refined
  uint32_t rem;       // keys still to take from inside [lo, hi]
  uint32_t inside;    // keys inside [lo, hi]
  uint32_t done;      // 1: [lo, hi] is final
  uint32_t n;         // scores in the row
  uint32_t pad[2];
};

__device__ __forceinline__ int row_len(const int32_t* q_pos, int row, int n_k) {
  int p = q_pos[row];
  p = p < -1 ? -1 : (p > n_k - 1 ? n_k - 1 : p);
  return p + 1;
}

// Exclusive prefix over the block of two counters (any block size that is a
// multiple of 64, up to 1024 threads).
template <int THREADS>
__device__ __forceinline__ void excl_scan2(uint32_t a, uint32_t b, uint32_t& ea, uint32_t& eb, uint32_t& ta,
                                           uint32_t& tb, uint32_t* red) {
  constexpr int W = THREADS / 64;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t ia = a, ib = b;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t xa = __shfl_up(ia, o, 64), xb = __shfl_up(ib, o, 64);
    if (lane >= o) { ia += xa; ib += xb; }
  }
  if (lane == 63) { red[wave] = ia; red[W + wave] = ib; }
  __syncthreads();
  uint32_t pa = 0, pb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int w = 0; w < W; ++w) {
    const uint32_t xa = red[w], xb = red[W + w];
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

// The 4 keys of positions p0..p0+3 (p0 a multiple of 4; key 0 past the row
// end: below every real key).  Branch-free, so that a thread's loads are all
// in flight together: the address is clamped into the row and the keys past
// its end masked.  With 16-byte aligned rows and a row stride that is a
// multiple of 4, a vector at p0 <= n - 1 stays inside the row's storage.
template <bool ALIGNED>
__device__ __forceinline__ u32x4 load_keys4(const float* __restrict__ src, int p0, int n) {
  f32x4 x;
  if constexpr (ALIGNED) {
    x = *reinterpret_cast<const f32x4*>(src + min(p0, (n - 1) & ~3));
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = src[min(p0 + e, n - 1)];
  }
  u32x4 k;
#pragma unroll
  for (int e = 0; e < 4; ++e) k[e] = p0 + e < n ? score_key(x[e]) : 0u;
  return k;
}

constexpr int kSteps = kChunk / (4 * kTkmThreads);   // 8 vectors of 4 scores per thread

// Every key of this thread in chunk [base, base + kChunk): vector i covers
// positions base + 4 kTkmThreads i + 4 tid + 0..3.
template <bool ALIGNED>
__device__ __forceinline__ void load_chunk(const float* __restrict__ src, int base, int n, u32x4 (&k)[kSteps]) {
#pragma unroll
  for (int i = 0; i < kSteps; ++i) k[i] = load_keys4<ALIGNED>(src, base + i * 4 * kTkmThreads + 4 * (int)threadIdx.x, n);
}

__global__ void tkm_init(RowState* __restrict__ st, uint32_t* __restrict__ ghist, const int32_t* __restrict__ q_pos,
                         int n_k, int K) {
  const int row = blockIdx.x;
  uint32_t* h = ghist + (int64_t)row * kTkmBins;
  for (int b = threadIdx.x; b < kTkmBins; b += blockDim.x) h[b] = 0u;
  if (threadIdx.x == 0) {
    const int n = row_len(q_pos, row, n_k);
    RowState s{};
    s.lo = 0xFFFFFFFFu;
    s.hi = 0u;
    s.rem = (uint32_t)K;
    s.inside = (uint32_t)n;
    s.done = n <= K ? 1u : 0u;
    s.n = (uint32_t)n;
    st[row] = s;
  }
}

template <bool ALIGNED>
__global__ __launch_bounds__(kTkmThreads) void tkm_minmax(const float* __restrict__ scores, int64_t ld,
                                                          RowState* __restrict__ st) {
  __shared__ uint32_t red[2 * (kTkmThreads / 64)];
  const int row = blockIdx.y, c = blockIdx.x;
  const int n = (int)st[row].n;
  if (st[row].done) return;
  const int base = c * kChunk;
  if (base >= n) return;
  const float* src = scores + (int64_t)row * ld;
  uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
  u32x4 kc[kSteps];
  load_chunk<ALIGNED>(src, base, n, kc);
#pragma unroll
  for (int i = 0; i < kSteps; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kmin = min(kmin, kc[i][e] ? kc[i][e] : 0xFFFFFFFFu);
      kmax = max(kmax, kc[i][e]);
    }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
    kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, o, 64));
  }
  if (lane == 0) { red[wave] = kmin; red[kTkmThreads / 64 + wave] = kmax; }
  __syncthreads();
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 1; w < kTkmThreads / 64; ++w) {
      kmin = min(kmin, red[w]);
      kmax = max(kmax, red[kTkmThreads / 64 + w]);
    }
    kmin = min(kmin, red[0]);
    kmax = max(kmax, red[kTkmThreads / 64]);
    atomicMin(&st[row].lo, kmin);
    atomicMax(&st[row].hi, kmax);
  }
}

// Bins of the range [lo, hi]: bin = (key - lo) >> shift, at most 2048 bins.
__device__ __forceinline__ int range_shift(uint32_t lo, uint32_t hi) {
  const uint32_t width = hi - lo;
  const int bits = 32 - __clz(width);
  return bits > 11 ? bits - 11 : 0;
}

template <bool ALIGNED>
__global__ __launch_bounds__(kTkmThreads) void tkm_hist(const float* __restrict__ scores, int64_t ld,
                                                        const RowState* __restrict__ st, uint32_t* __restrict__ ghist) {
  __shared__ uint32_t h[kTkmBins];
  const int row = blockIdx.y, c = blockIdx.x;
  const RowState s = st[row];
  if (s.done) return;
  const int n = (int)s.n, base = c * kChunk;
  if (base >= n) return;
  const int shift = range_shift(s.lo, s.hi);
  const int nbins = (int)((s.hi - s.lo) >> shift) + 1;
  const float* src = scores + (int64_t)row * ld;
  u32x4 kc[kSteps];
  load_chunk<ALIGNED>(src, base, n, kc);
  for (int b = threadIdx.x; b < nbins; b += kTkmThreads) h[b] = 0u;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kSteps; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (kc[i][e] >= s.lo && kc[i][e] <= s.hi) atomicAdd(&h[(kc[i][e] - s.lo) >> shift], 1u);
  __syncthreads();
  uint32_t* g = ghist + (int64_t)row * kTkmBins;
  for (int b = threadIdx.x; b < nbins; b += kTkmThreads)
    if (h[b]) atomicAdd(&g[b], h[b]);
}

// One workgroup per row: the bin holding the rem-th largest key inside
// [lo, hi] becomes the new range; the histogram is cleared for the next round.
__global__ __launch_bounds__(256) void tkm_select(RowState* __restrict__ st, uint32_t* __restrict__ ghist, int K) {
  constexpr int BPT = kTkmBins / 256;
  __shared__ uint32_t red[8];
  __shared__ uint32_t pick[3];
  const int row = blockIdx.x, tid = threadIdx.x;
  const RowState s = st[row];
  if (s.done) return;
  const int shift = range_shift(s.lo, s.hi);
  const int nbins = (int)((s.hi - s.lo) >> shift) + 1;
  uint32_t* g = ghist + (int64_t)row * kTkmBins;
  uint32_t hb[BPT], hsum = 0;
#pragma unroll
  for (int e = 0; e < BPT; ++e) {
    const int b = BPT * tid + e;
    hb[e] = b < nbins ? g[b] : 0u;
    hsum += hb[e];
  }
  uint32_t ex, ex2, tot, tot2;
  excl_scan2<256>(hsum, 0u, ex, ex2, tot, tot2, red);
  uint32_t above = tot - (ex + hsum);   // keys in bins above this thread's bins
#pragma unroll
  for (int e = BPT - 1; e >= 0; --e) {
    const int b = BPT * tid + e;
    if (b < nbins && above < s.rem && s.rem <= above + hb[e]) {
      pick[0] = (uint32_t)b;
      pick[1] = above;
      pick[2] = hb[e];
    }
    above += hb[e];
  }
  __syncthreads();
  for (int b = tid; b < kTkmBins; b += 256) g[b] = 0u;
  if (tid == 0) {
    const uint32_t b = pick[0];
    const uint64_t nlo = (uint64_t)s.lo + ((uint64_t)b << shift);
    const uint64_t nhi = nlo + ((uint64_t)1 << shift) - 1;
    RowState t = s;
    t.lo = (uint32_t)nlo;
    t.hi = (uint32_t)(nhi < (uint64_t)s.hi ? nhi : (uint64_t)s.hi);
    t.rem = s.rem - pick[1];
    t.inside = pick[2];
    t.done = (t.inside <= (uint32_t)K || t.lo == t.hi) ? 1u : 0u;
    st[row] = t;
  }
}

// Per chunk, in position order: positions with key > hi to abuf, (position,
// key) with lo <= key <= hi to cbuf (the first K of the chunk), and the two
// counts.
template <bool ALIGNED>
__global__ __launch_bounds__(kTkmThreads) void tkm_collect(const float* __restrict__ scores, int64_t ld,
                                                           const RowState* __restrict__ st, int nch, int K,
                                                           int32_t* __restrict__ abuf, uint2* __restrict__ cbuf,
                                                           uint32_t* __restrict__ cnt) {
  __shared__ uint32_t red[2 * (kTkmThreads / 64)];
  const int row = blockIdx.y, c = blockIdx.x;
  const RowState s = st[row];
  const int n = (int)s.n, base = c * kChunk;
  uint32_t* my_cnt = cnt + ((int64_t)row * nch + c) * 2;
  if (n <= K || base >= n) {
    if (threadIdx.x == 0) my_cnt[0] = my_cnt[1] = 0u;
    return;
  }
  const float* src = scores + (int64_t)row * ld;
  int32_t* ab = abuf + ((int64_t)row * nch + c) * K;
  uint2* cb = cbuf + ((int64_t)row * nch + c) * K;
  uint32_t na = 0, nc = 0;
  // vectors i + 1 and i + 2 are loaded while vector i is ranked
  u32x4 k_next = load_keys4<ALIGNED>(src, base + 4 * (int)threadIdx.x, n);
  u32x4 k_next2 = load_keys4<ALIGNED>(src, base + 4 * kTkmThreads + 4 * (int)threadIdx.x, n);
  for (int i = 0; i < kSteps; ++i) {
    const int p0 = base + i * 4 * kTkmThreads + 4 * threadIdx.x;
    if (base + i * 4 * kTkmThreads >= n) break;   // uniform
    const u32x4 k = k_next;
    k_next = k_next2;
    if (i + 2 < kSteps) k_next2 = load_keys4<ALIGNED>(src, p0 + 8 * kTkmThreads, n);
    uint32_t a = 0, b = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a += k[e] > s.hi;
      b += k[e] >= s.lo && k[e] <= s.hi;
    }
    uint32_t ea, eb, ta, tb;
    excl_scan2<kTkmThreads>(a, b, ea, eb, ta, tb, red);
    ea += na;
    eb += nc;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (k[e] > s.hi) {   // fewer than K above hi in the whole row
        if (ea < (uint32_t)K) ab[ea] = p0 + e;
        ++ea;
      }
      else if (k[e] >= s.lo && k[e] <= s.hi) {
        if (eb < (uint32_t)K) cb[eb] = make_uint2((uint32_t)(p0 + e), k[e]);
        ++eb;
      }
    }
    na += ta;
    nc += tb;
  }
  if (threadIdx.x == 0) {
    my_cnt[0] = na;
    my_cnt[1] = min(nc, (uint32_t)K);
  }
}

// First index in a[0..len) whose value is >= x (a ascending).
__device__ __forceinline__ int lower_bound_lds(const int32_t* a, int len, int32_t x) {
  int lo = 0, hi = len;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] < x) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

__global__ __launch_bounds__(kFinalThreads) void tkm_final(const RowState* __restrict__ st, int nch, int K,
                                                           const int32_t* __restrict__ abuf,
                                                           const uint2* __restrict__ cbuf,
                                                           const uint32_t* __restrict__ cnt,
                                                           int32_t* __restrict__ idx) {
  __shared__ int32_t s_above[SMA_MAX_TOPK_DEV];
  __shared__ int32_t s_sel[SMA_MAX_TOPK_DEV];
  __shared__ uint32_t s_ckey[SMA_MAX_TOPK_DEV];     // candidate keys (sorted descending below)
  __shared__ uint32_t s_cidx[SMA_MAX_TOPK_DEV];     // their index in the position-ordered list
  __shared__ int32_t s_cpos[SMA_MAX_TOPK_DEV];
  __shared__ uint32_t s_flag[SMA_MAX_TOPK_DEV];
  __shared__ uint32_t red[2 * (kFinalThreads / 64)];
  __shared__ uint32_t s_goa[kFinalThreads], s_goc[kFinalThreads];   // a chunk group's list offsets
  const int row = blockIdx.x, tid = threadIdx.x;
  const RowState s = st[row];
  const int n = (int)s.n;
  int32_t* out = idx + (int64_t)row * K;
  if (n <= K) {
    for (int e = tid; e < K; e += kFinalThreads) out[e] = e < n ? e : -1;
    return;
  }
  // Concatenate the chunks' lists (chunks in position order): positions
  // above hi, then the candidates; with one key left (lo == hi) only the
  // first `rem` candidates can be taken.  The chunks' counts are read and
  // scanned kFinalThreads at a time, so every chunk's offsets are known
  // before any entry moves.
  const uint32_t* rc = cnt + (int64_t)row * nch * 2;
  const uint32_t want_c = s.lo == s.hi ? s.rem : (uint32_t)K;
  uint32_t run_a = 0, run_c = 0;   // entries of earlier chunk groups
  for (int g0 = 0; g0 < nch; g0 += kFinalThreads) {
    const int c = g0 + tid;
    const uint32_t na = c < nch ? rc[2 * c] : 0u, nc = c < nch ? rc[2 * c + 1] : 0u;
    uint32_t ea, ec, ta, tc;
    excl_scan2<kFinalThreads>(na, nc, ea, ec, ta, tc, red);
    if (c < nch) {
      s_goa[tid] = run_a + ea;
      s_goc[tid] = run_c + ec;
    }
    __syncthreads();
    // Entry g of the group's list lies in the last chunk whose offset is
    // <= g (an empty chunk shares its offset with the next one); threads
    // take entries of the whole group, so all the loads are in flight at once.
    const int gn = min(kFinalThreads, nch - g0);
    auto chunk_of = [&](const uint32_t* off, uint32_t g) {
      int lo = 0, hi = gn - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= g) lo = mid;
        else hi = mid - 1;
      }
      return lo;
    };
    const uint32_t a_end = min(run_a + ta, (uint32_t)K);
    for (uint32_t g = run_a + tid; g < a_end; g += kFinalThreads) {
      const int k = chunk_of(s_goa, g);
      s_above[g] = abuf[((int64_t)row * nch + g0 + k) * K + (g - s_goa[k])];
    }
    const uint32_t c_end = min(run_c + tc, want_c);
    for (uint32_t g = run_c + tid; g < c_end; g += kFinalThreads) {
      const int k = chunk_of(s_goc, g);
      const uint2 v = cbuf[((int64_t)row * nch + g0 + k) * K + (g - s_goc[k])];
      s_cpos[g] = (int32_t)v.x;
      s_ckey[g] = v.y;
    }
    run_a += ta;
    run_c += tc;
    __syncthreads();
  }
  const int A = (int)min(run_a, (uint32_t)K);   // = K - rem
  const int C = (int)min(run_c, want_c);
  const int R = min((int)s.rem, K - A);              // candidates taken (= rem)
  // ---- which candidates are taken ----
  if (s.lo == s.hi) {
    // all candidates share the key: the first R in position order
    for (int j = tid; j < C; j += kFinalThreads) s_flag[j] = j < R ? 1u : 0u;
  } else {
    // rank the C <= K candidates by (key descending, position ascending)
    // with a bitonic sort of (key, index) over the next power of two
    int P = 1;
    while (P < C) P <<= 1;
    for (int j = tid; j < P; j += kFinalThreads) {
      if (j >= C) { s_ckey[j] = 0u; s_cidx[j] = 0xFFFFFFFFu; }
      else s_cidx[j] = (uint32_t)j;
    }
    __syncthreads();
    // "a before b": larger key first, then smaller index (= lower position)
    auto before = [&](uint32_t ka, uint32_t ia, uint32_t kb, uint32_t ib) {
      return ka > kb || (ka == kb && ia < ib);
    };
    for (int size = 2; size <= P; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int j = tid; j < P; j += kFinalThreads) {
          const int partner = j ^ stride;
          if (partner > j) {
            const bool up = (j & size) == 0;
            const uint32_t ka = s_ckey[j], ia = s_cidx[j], kb = s_ckey[partner], ib = s_cidx[partner];
            const bool swap = up ? before(kb, ib, ka, ia) : before(ka, ia, kb, ib);
            if (swap) {
              s_ckey[j] = kb; s_cidx[j] = ib;
              s_ckey[partner] = ka; s_cidx[partner] = ia;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int j = tid; j < C; j += kFinalThreads) s_flag[j] = 0u;
    __syncthreads();
    for (int j = tid; j < R; j += kFinalThreads)
      if (s_cidx[j] < (uint32_t)C) s_flag[s_cidx[j]] = 1u;
  }
  __syncthreads();
  // ---- taken candidates, still in position order ----
  {
    uint32_t done_cnt = 0;
    for (int b0 = 0; b0 < C; b0 += kFinalThreads) {
      const int j = b0 + tid;
      const uint32_t f = j < C ? s_flag[j] : 0u;
      uint32_t ef, e2, tf, t2;
      excl_scan2<kFinalThreads>(f, 0u, ef, e2, tf, t2, red);
      if (f && done_cnt + ef < (uint32_t)K) s_sel[done_cnt + ef] = s_cpos[j];
      done_cnt += tf;
    }
  }
  __syncthreads();
  // ---- merge the two ascending lists into the output ----
  for (int i = tid; i < A; i += kFinalThreads) {
    const int r = i + lower_bound_lds(s_sel, R, s_above[i]);
    if (r < K) out[r] = s_above[i];
  }
  for (int j = tid; j < R; j += kFinalThreads) {
    const int r = j + lower_bound_lds(s_above, A, s_sel[j]);
    if (r < K) out[r] = s_sel[j];
  }
}

}  // namespace

size_t topk_multi_bytes(int32_t n_q, int64_t n_k, int32_t top_k) {
  if (n_q <= 0 || n_k <= 0 || top_k <= 0) return 0;
  const int64_t nch = (n_k + kChunk - 1) / kChunk;
  auto al = [](size_t b) { return (b + 255) / 256 * 256; };
  return al((size_t)n_q * sizeof(RowState)) + al((size_t)n_q * kTkmBins * 4) + al((size_t)n_q * nch * 2 * 4) +
         al((size_t)n_q * nch * top_k * 4) + al((size_t)n_q * nch * top_k * 8);
}

hipError_t launch_topk_multi(const TopkArgs& A, void* ws, hipStream_t st) {
  if (A.n_q <= 0) return hipSuccess;
  const int nch = (int)((A.n_k + kChunk - 1) / kChunk);
  auto al = [](size_t b) { return (b + 255) / 256 * 256; };
  uint8_t* p = static_cast<uint8_t*>(ws);
  RowState* state = reinterpret_cast<RowState*>(p);
  p += al((size_t)A.n_q * sizeof(RowState));
  uint32_t* ghist = reinterpret_cast<uint32_t*>(p);
  p += al((size_t)A.n_q * kTkmBins * 4);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(p);
  p += al((size_t)A.n_q * nch * 2 * 4);
  int32_t* abuf = reinterpret_cast<int32_t*>(p);
  p += al((size_t)A.n_q * nch * A.top_k * 4);
  uint2* cbuf = reinterpret_cast<uint2*>(p);
  const bool aligned = (reinterpret_cast<uintptr_t>(A.scores) % 16 == 0) && (A.ld % 4 == 0);
  const dim3 grid2((unsigned)nch, (unsigned)A.n_q);
  hipLaunchKernelGGL(tkm_init, dim3((unsigned)A.n_q), dim3(256), 0, st, state, ghist, A.q_pos, (int)A.n_k, A.top_k);
#define SMA_TKM(KERNEL, ...)                                                                      \
  if (aligned) hipLaunchKernelGGL(KERNEL<true>, grid2, dim3(kTkmThreads), 0, st, __VA_ARGS__);   \
  else hipLaunchKernelGGL(KERNEL<false>, grid2, dim3(kTkmThreads), 0, st, __VA_ARGS__);
  SMA_TKM(tkm_minmax, A.scores, A.ld, state)
  for (int round = 0; round < 3; ++round) {
    SMA_TKM(tkm_hist, A.scores, A.ld, state, ghist)
    hipLaunchKernelGGL(tkm_select, dim3((unsigned)A.n_q), dim3(256), 0, st, state, ghist, A.top_k);
  }
  SMA_TKM(tkm_collect, A.scores, A.ld, state, nch, A.top_k, abuf, cbuf, cnt)
#undef SMA_TKM
  hipLaunchKernelGGL(tkm_final, dim3((unsigned)A.n_q), dim3(kFinalThreads), 0, st, state, nch, A.top_k, abuf, cbuf,
                     cnt, A.idx);
  return hipGetLastError();
}

}  // namespace sma
