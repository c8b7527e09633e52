// One DCP rank's share of sparse MLA and the log-sum-exp merge of the
// ranks' partial results (GLM-5.3 part 2, section "DCP : sharder aussi le
// cache KV": tokens are dealt round-robin over the ranks, so rank r stores
// tokens r, r + P, ...; in decode each rank attends over its own shard and
// the partial results are merged by their log-sum-exp).
//
//  * dcp_local_idx_kernel: from a query's global selection (ascending token
//    positions, -1 padding) keep the tokens rank r stores, as its local rows
//    s / P, in order, then -1 padding; the sparse-MLA kernels then run on the
//    rank's shard unchanged, writing fp32 partials and their lse.
//  * lse_merge_kernel: o = sum_r exp(lse_r - L) o_r with L = log sum_r
//    exp(lse_r); an all-empty (query, head) gives o = 0 and L = -inf.
#include "sma_device.h"
#include "sma_launch.h"

namespace sma {

constexpr int kDcpThreads = 256;
constexpr int kDcpPer = SMA_MAX_TOPK_DEV / kDcpThreads;   // 8 entries per thread

// One workgroup per query row; thread t scans entries [8t, 8t + 8).
__global__ __launch_bounds__(kDcpThreads) void dcp_local_idx_kernel(const int32_t* __restrict__ idx, int K,
                                                                    int rank, int P, int64_t n_k_local,
                                                                    int32_t* __restrict__ local) {
  __shared__ uint32_t s_wave[kDcpThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int32_t* in = idx + (int64_t)blockIdx.x * K;
  int32_t* out = local + (int64_t)blockIdx.x * K;
  int32_t v[kDcpPer];
#pragma unroll
  for (int j = 0; j < kDcpPer; ++j) v[j] = in[min(kDcpPer * tid + j, K - 1)];   // all in flight together
  uint32_t keep = 0, cnt = 0;
#pragma unroll
  for (int j = 0; j < kDcpPer; ++j) {
    const int e = kDcpPer * tid + j;
    const int32_t x = e < K ? v[j] : -1;
    const bool mine = x >= 0 && x % P == rank && (int64_t)(x / P) < n_k_local;
    v[j] = mine ? x / P : -1;
    keep |= (uint32_t)mine << j;
    cnt += mine;
  }
  // exclusive prefix of the counts over the workgroup, in entry order
  uint32_t incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = (uint32_t)__shfl_up((int)incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  uint32_t before = incl - cnt, total = 0;
#pragma unroll
  for (int w = 0; w < kDcpThreads / 64; ++w) {
    const uint32_t x = s_wave[w];
    before += w < wave ? x : 0u;
    total += x;
  }
#pragma unroll
  for (int j = 0; j < kDcpPer; ++j)
    if ((keep >> j) & 1u) out[before++] = v[j];
  for (int e = (int)total + tid; e < K; e += kDcpThreads) out[e] = -1;
}

// One workgroup per (query, group of 8 heads), so that a decode-sized batch
// still spreads over the CUs: the per-(rank, head) weights go to LDS, then
// each thread merges 16-byte pieces of the group's [8, 512] outputs.
constexpr int kMergeHeads = 8;
template <bool OUT_F32>
__global__ __launch_bounds__(kDcpThreads) void lse_merge_kernel(const float* __restrict__ parts,
                                                                const float* __restrict__ lses, int n_part,
                                                                int n_q, void* __restrict__ out,
                                                                float* __restrict__ lse_out) {
  __shared__ float s_w[kMaxMergeParts][kMergeHeads];
  const int tid = threadIdx.x;
  const int qi = blockIdx.x / (kHeads / kMergeHeads), h0 = kMergeHeads * (blockIdx.x % (kHeads / kMergeHeads));
  const int64_t part_stride = (int64_t)n_q * kHeads * kDv;
  // the (rank, head) lse values, one per thread (head t & 7, rank t >> 3 and
  // t >> 3 + 32), so that they arrive in one or two round trips
  for (int i = tid; i < n_part * kMergeHeads; i += kDcpThreads) {
    const int r = i / kMergeHeads, hh = i % kMergeHeads;
    s_w[r][hh] = lses[((int64_t)r * n_q + qi) * kHeads + h0 + hh];
  }
  __syncthreads();
  if (tid < kMergeHeads) {
    const int h = h0 + tid;
    float m = -INFINITY;
    for (int r = 0; r < n_part; ++r) m = fmaxf(m, s_w[r][tid]);
    float s = 0.f;
    for (int r = 0; r < n_part; ++r) {
      const float l = s_w[r][tid];
      const float a = m == -INFINITY || l == -INFINITY ? 0.f : __expf(l - m);
      s_w[r][tid] = a;
      s += a;
    }
    const float inv = s > 0.f ? 1.f / s : 0.f;
    for (int r = 0; r < n_part; ++r) s_w[r][tid] *= inv;
    if (lse_out) lse_out[(int64_t)qi * kHeads + h] = s > 0.f ? m + __logf(s) : -INFINITY;
  }
  __syncthreads();
  // Each thread merges four 16-byte pieces (f = tid + 256i, head 2i + (tid
  // >> 7) of the group); the ranks' pieces are loaded four ranks at a time
  // (clamped rank index, all in flight together), and a rank of zero weight
  // adds nothing.
  constexpr int kPieces = kMergeHeads * kDv / 4 / kDcpThreads, kGroup = 4;
  const int64_t base = ((int64_t)qi * kHeads + h0) * kDv;   // first float of the group
  f32x4 acc[kPieces];
#pragma unroll
  for (int i = 0; i < kPieces; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int r0 = 0; r0 < n_part; r0 += kGroup) {
    f32x4 v[kGroup][kPieces];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const f32x4* src = reinterpret_cast<const f32x4*>(parts + min(r0 + j, n_part - 1) * part_stride + base);
#pragma unroll
      for (int i = 0; i < kPieces; ++i) v[j][i] = src[tid + kDcpThreads * i];
    }
#pragma unroll
    for (int j = 0; j < kGroup; ++j)
#pragma unroll
      for (int i = 0; i < kPieces; ++i) {
        const float wr = r0 + j < n_part ? s_w[r0 + j][(tid + kDcpThreads * i) / (kDv / 4)] : 0.f;
        if (wr != 0.f) acc[i] += wr * v[j][i];
      }
  }
#pragma unroll
  for (int i = 0; i < kPieces; ++i) {
    const int f = tid + kDcpThreads * i;
    if constexpr (OUT_F32) {
      reinterpret_cast<f32x4*>(static_cast<float*>(out) + base)[f] = acc[i];
    } else {
      reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + base)[f] =
          u32x2{pack_bf16x2(acc[i][0], acc[i][1]), pack_bf16x2(acc[i][2], acc[i][3])};
    }
  }
}

hipError_t launch_dcp_local_idx(const int32_t* idx, int n_q, int K, int rank, int P, int64_t n_k_local,
                                int32_t* local, hipStream_t st) {
  if (n_q <= 0) return hipSuccess;
  hipLaunchKernelGGL(dcp_local_idx_kernel, dim3((unsigned)n_q), dim3(kDcpThreads), 0, st, idx, K, rank, P,
                     n_k_local, local);
  return hipGetLastError();
}

hipError_t launch_lse_merge(const float* parts, const float* lses, int n_part, int n_q, void* out, bool out_f32,
                            float* lse_out, hipStream_t st) {
  if (n_q <= 0) return hipSuccess;
  const dim3 grid((unsigned)n_q * (kHeads / kMergeHeads));
  if (out_f32)
    hipLaunchKernelGGL((lse_merge_kernel<true>), grid, dim3(kDcpThreads), 0, st, parts, lses, n_part, n_q, out,
                       lse_out);
  else
    hipLaunchKernelGGL((lse_merge_kernel<false>), grid, dim3(kDcpThreads), 0, st, parts, lses, n_part, n_q, out,
                       lse_out);
  return hipGetLastError();
}

}  // namespace sma
