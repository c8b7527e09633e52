// Sparse MLA gather-attention kernels (gfx950), absorbed / "MQA" mode.
//
// All 64 heads of one query attend over the query's selected latent rows:
// z = tau * q_h . kv_s[0:576], softmax over the selected set, o_h = sum_s
// p_s kv_s[0:512] (GLM-5.3 part 2, "PCP : répartir les tokens, pas les
// têtes" and footnote 1: one KV row read serves every head; QK over 576, PV
// over 512).
//
// One kernel (sparse_mla_kernel) computes it for three KV row formats:
// bf16 rows (576 x 2 bytes); per-token FP8 rows (576 e4m3 codes, one fp32
// scale per row in a separate array), whose scale stays out of the bf16
// operands (it multiplies the row's logit and softmax weight, so the codes
// widen to bf16 exactly); and FlashMLA's 656-byte fp8_ds_mla row (512 codes,
// four fp32 scales of 128 dims each, 64 bf16 rope dims; GLM-5.3 part 2,
// footnote 1, names it), whose codes are widened as bf16(code x block
// scale), one rounding per element, so QK and PV run as for bf16 rows.  One
// 2-wave workgroup per query (or per slice of a query's rows on small
// batches, merged by mla_merge_kernel) splits both contractions by dims,
// gathers with direct global->LDS loads and uses v_mfma_f32_32x32x16_bf16;
// its design is described where it is defined.
// Writing the products transposed puts one head per lane column in both
// accumulators, so the softmax statistics of a head and the output rows
// they scale live in the same lanes.
#include <algorithm>
#include <type_traits>

#include "sma_device.h"
#include "sma_launch.h"

namespace sma {

constexpr int kMlaRows = 32;                // gathered rows per tile
// Split partial of one (query, slice): O [64][512] unnormalised, then the
// per-head exponent reference m (log2 domain) and sum l.
constexpr int kMlaPartFloats = kHeads * kDv + 2 * kHeads;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef int i32x2v __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2v lds_i32x2;

// Log-sum-exp merge of the n_split partials of each query: with
// M = max_s m_s, out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s and
// lse = (M + log2 of that sum) * ln 2.  A 256-thread workgroup merges 4
// heads of one query (16 workgroups per query, so a 64-query batch keeps
// 1,024 workgroups busy): thread t takes head 4 blockIdx.y + (t >> 6) and
// dims 8 (t & 63) .. + 7, so consecutive threads read consecutive 32 bytes
// of each partial.
constexpr int kMergeHeads = 4;

template <bool OUT_F32>
__global__ __launch_bounds__(256) void mla_merge_kernel(const float* __restrict__ part, int n_split,
                                                        void* __restrict__ out, float* __restrict__ lse) {
  constexpr int kMaxSplit = 16, kGroup = 4;
  const int qi = blockIdx.x, h = kMergeHeads * blockIdx.y + (threadIdx.x >> 6), c8 = threadIdx.x & 63;
  const float* base = part + (int64_t)qi * n_split * kMlaPartFloats;
  // Every load below takes a clamped split index and is issued before any
  // result is used, so the references and sums arrive in one round trip and
  // the outputs in one per group of four slices.
  float m[kMaxSplit], ls[kMaxSplit];
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s) {
    const float* ps = base + min(s, n_split - 1) * kMlaPartFloats + kHeads * kDv;
    m[s] = ps[h];
    ls[s] = ps[kHeads + h];
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s) M = s < n_split ? fmaxf(M, m[s]) : M;
  float wgt[kMaxSplit], L = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxSplit; ++s) {
    wgt[s] = s >= n_split || m[s] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[s] - M);
    L += wgt[s] * ls[s];
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  f32x4 acc0 = f32x4{0.f, 0.f, 0.f, 0.f}, acc1 = acc0;
  for (int s0 = 0; s0 < n_split; s0 += kGroup) {
    f32x4 v[kGroup][2];
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const float* src = base + min(s0 + j, n_split - 1) * kMlaPartFloats + h * kDv + 8 * c8;
      v[j][0] = *reinterpret_cast<const f32x4*>(src);
      v[j][1] = *reinterpret_cast<const f32x4*>(src + 4);
    }
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      float wj = 0.f;
#pragma unroll
      for (int s = 0; s < kMaxSplit; ++s) wj = s == s0 + j ? wgt[s] : wj;   // 0 past n_split
      acc0 += wj * v[j][0];
      acc1 += wj * v[j][1];
    }
  }
  acc0 *= inv;
  acc1 *= inv;
  const int64_t o_off = ((int64_t)qi * kHeads + h) * kDv + 8 * c8;
  if constexpr (OUT_F32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + o_off) = acc0;
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + o_off + 4) = acc1;
  } else {
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + o_off) =
        u32x4{pack_bf16x2(acc0[0], acc0[1]), pack_bf16x2(acc0[2], acc0[3]), pack_bf16x2(acc1[0], acc1[1]),
              pack_bf16x2(acc1[2], acc1[3])};
  }
  if (lse && c8 == 0)
    lse[(int64_t)qi * kHeads + h] = L > 0.f ? (M + __log2f(L)) * 0.69314718055994531f : -INFINITY;
}

// ---------------------------------------------------------------------------
// Helpers of the bf16 kernel below: direct global->LDS loads, hand-kept
// vmcnt bookkeeping, and MFMAs with VGPR accumulators.
// ---------------------------------------------------------------------------
constexpr float kRefGap = 64.f;                         // log2 units
constexpr int kDmaRowB = kDqk * 2;                      // 1152
constexpr int kDmaTileB = kMlaRows * kDmaRowB;          // 36864

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef float f32x16v_t __attribute__((ext_vector_type(16)));

// One 16-byte-per-lane global->LDS load: lane l's 16 bytes land at LDS byte
// address lds_base + 16*l.  Issued from inline assembly so that the
// compiler's wait-count insertion does not treat it as aliasing the ring
// slots being read; completion is tracked by hand with wait_vmcnt<>.
__device__ __forceinline__ void dma_load16(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gaddr), "s"(lds_base)
               : "memory", "m0");
}
// The same from gaddr + OFF (OFF < 4096), with OFF in the instruction's
// offset field so that loads along one row share an address register.  The
// instruction adds its offset to the LDS address as well, so M0 is lowered
// by OFF (lds_base >= OFF).
template <int OFF>
__device__ __forceinline__ void dma_load16_at(const void* gaddr, uint32_t lds_base) {
  static_assert(OFF >= 0 && OFF < 4096, "global instruction offset range");
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off offset:%2" ::"v"(gaddr), "s"(lds_base - OFF),
               "i"(OFF)
               : "memory", "m0");
}

// v_mfma_f32_32x32x16_bf16 with its accumulator in VGPRs.  The compiler
// emits every MFMA builtin of a kernel that also uses AGPRs in the AGPR
// form; the output accumulators fill the AGPR file, so the QK partial sums
// are formed through these instead.  Being opaque to the compiler's hazard
// recognizer, they carry their own wait states, counted from the MFMA
// dependency table of AMD's CDNA3/CDNA4 instruction-set reference (the
// required independent instructions between a VALU write and an XDL read of
// the same VGPR, and between an XDL write and a VALU / LDS read of its
// result, by pass count): two before each MFMA (a VALU write of an A/B
// register just before it) and, in drain, 24 after the last one before any
// VALU or LDS instruction reads the result (an 8-pass XDL op needs 11).  A
// dependent chain through the same accumulator (SrcC = the previous
// result) needs none.
__device__ __forceinline__ void mfma32_vgpr_first(f32x16v_t& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_vgpr(f32x16v_t& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma32_vgpr_drain(f32x16v_t& x, f32x16v_t& y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x), "+v"(y));
}
// Wait states after the last MFMA into x when one more MFMA is issued
// before x is read (16 + 1 >= 11).
__device__ __forceinline__ void mfma32_vgpr_drain1(f32x16v_t& x) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(x));
}

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

// bf16 KV kernel.  One 2-wave workgroup per query, two workgroups per CU
// (one wave per SIMD).  The two waves split every contraction by dims, so
// each byte of a gathered tile is read from LDS by exactly one wave:
//   QK: wave d holds Q for all 64 heads over dims 288d..288d+287 (144
//       VGPRs) and forms a partial S^T[32 rows x 64 heads] with
//       v_mfma_f32_32x32x16_bf16 (A = K rows, B = Q);  the partner's
//       half-sum for the heads this wave owns arrives through LDS;
//   softmax: wave d owns heads 32d..32d+31;  its bf16 P goes to the partner
//       through LDS;
//   PV: wave d accumulates O^T[dims 256d..256d+255 x 64 heads] (256 AGPRs)
//       with A = V^T read by ds_read_b64_tr_b16 and B = P.
// Softmax weights use a fixed per-head reference (below), so the output
// registers are only ever written by MFMAs.
//
// Tile layout (32 rows x 576 dims, 36 KiB): a 1-KiB block holds 8 rows x
// 128 bytes, block (rg, cg) = row group r >> 3 and 128-byte chunk group at
// (4 cg + rg) KiB.  Inside a block row r takes 128 bytes at 128 (r & 7), and
// its 16-byte chunk c sits at slot (c & 7) ^ swz(r), swz(r) = bit-reverse of
// the 3 bits (r >> 1) & 7.  A direct global->LDS load fills one block: eight
// consecutive lanes fetch the 128 contiguous bytes of one row (each lane the
// chunk that belongs at its 16 bytes), which the memory path coalesces far
// better than 16-byte pieces of 16 rows.  Wave d gathers row groups 2d and
// 2d+1: two indices per lane per tile.  A 16-byte read serves 16 lanes per
// cycle and a transposed 8-byte read 32 lanes; the swizzle puts each such
// group of the K operand reads and of the V^T reads on distinct banks, and
// the reads need four base registers each plus immediate offsets.  The rope
// chunk group (cg 8, bytes 32768..36863) is dead after QK and carries the
// S/P exchange of one direction; a 4-KiB buffer carries the other.
//
// Entries are used in their given order without compaction: invalid ones
// (negative, past n_k or past top_k) gather row 0 and are masked out of the
// softmax by a per-tile row mask.
constexpr int kPairThreads = 128;
constexpr int kPairLoads = kDmaTileB / 1024 / 2;   // 18 one-KiB loads per wave per tile
constexpr int kPairKs = kDqk / 16 / 2;             // 18 k-steps of QK per wave
constexpr int kPairMt = kDv / 32 / 2;              // 8 M-tiles of PV per wave
constexpr int kRopeOff = kDv * 2 / 32 * 1024;      // 32768: first byte of the rope blocks
constexpr int kIdxChunk = 256;                     // entries per staged index chunk (8 tiles)

// One 4-byte-per-lane global->LDS load (lane l's word lands at lds_base + 4l).
__device__ __forceinline__ void dma_load4(const void* gaddr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dword %0, off" ::"v"(gaddr), "s"(lds_base)
               : "memory", "m0");
}

typedef f32x16v_t f32x16v;

// swz(r): bit-reverse of (r >> 1) & 7 (the 16-byte slot swizzle of row r).
__device__ __forceinline__ int tile_swz(int r) {
  const int u = (r >> 1) & 7;
  return ((u & 1) << 2) | (u & 2) | ((u >> 2) & 1);
}
__device__ __forceinline__ constexpr int tile_block(int rg, int cg) { return (4 * cg + rg) * 1024; }

// Eight e4m3 codes (bytes 0..7 of lo, hi) -> eight bf16 in byte order,
// exactly (v_cvt_scalef32_pk_bf16_fp8 at scale 1: every e4m3 value is a bf16
// value; at other scales the instruction does not round to nearest).
__device__ __forceinline__ bf16x8 widen8(uint32_t lo, uint32_t hi) {
  u32x4 w;
  w[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, false));
  w[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.f, true));
  w[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, false));
  w[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.f, true));
  return __builtin_bit_cast(bf16x8, w);
}

// Widen the 16-code pieces P0 .. P0 + 2 NI - 1 of every row of an
// fp8_ds_mla tile (dims 16 P0 .. 16 (P0 + 2 NI) - 1) from its staging slot
// into the bf16 tile, each code times its row's scale of its 128-dim block
// (bsc = the row's four scales), rounded once to bf16.  The staging slot
// holds piece c of row r at byte 1024 (c >> 1) + 512 (c & 1) + 16 r (the
// gather's load k = c >> 1, lane 32 (c & 1) + r), so lane l (row l & 31,
// pieces P0 + (l >> 5) + 2i) reads 16 bytes at 1024 (P0 / 2 + i) + 16 l;
// those pieces lie in block (P0 + 2i) >> 3 (P0 + 2i is even, so adding
// l >> 5 stays in the block); bf16 chunk cc = 2c + hh of row r goes to its
// block (r >> 3, cc >> 3) = (r >> 3, P0 / 4 + i / 2) at slot (cc & 7) ^
// swz(r), cc & 7 = 4 (i & 1) + 2 (l >> 5) + hh.
template <int P0, int NI>
__device__ __forceinline__ void widen_ds_dims(const uint8_t* stage, uint8_t* tile, int lane, f32x4 bsc) {
  static_assert(P0 % 4 == 0, "pieces start at a chunk group");
  const int r = lane & 31, g = lane >> 5, sw = tile_swz(r);
  uint8_t* rowp = tile + tile_block(r >> 3, 0) + 128 * (r & 7);
  int off[2][2];
#pragma unroll
  for (int ip = 0; ip < 2; ++ip)
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) off[ip][hh] = 16 * ((4 * ip + 2 * g + hh) ^ sw);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(stage + 1024 * (P0 / 2 + i) + 16 * lane);
    const float sc = bsc[((P0 + 2 * i) >> 3) & 3];
    uint32_t w[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[e], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)v[e], true);
      w[2 * e] = pack_bf16x2(lo[0] * sc, lo[1] * sc);
      w[2 * e + 1] = pack_bf16x2(hi[0] * sc, hi[1] * sc);
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
      *reinterpret_cast<u32x4*>(rowp + 4096 * (P0 / 4 + i / 2) + off[i & 1][hh]) =
          u32x4{w[4 * hh], w[4 * hh + 1], w[4 * hh + 2], w[4 * hh + 3]};
  }
}

// KV row formats.
constexpr int kKvBf16 = 0;     // 576 bf16 dims (1,152 bytes)
constexpr int kKvFp8Row = 1;   // 576 e4m3 codes; one fp32 scale per row in a separate array
constexpr int kKvFp8Ds = 2;    // fp8_ds_mla: 512 codes, 4 fp32 block scales, 64 bf16 rope dims
constexpr int kDsRowB = 656;
constexpr int kDsScaleOff = 512, kDsRopeOff = 528;   // byte offsets inside a 656-byte row

// FP8 rows (kKvFp8Row, kKvFp8Ds).  A tile's codes are gathered by the same
// direct global->LDS loads into one of two staging slots (half the bytes of
// a bf16 tile), the row scales beside them.
//  * kKvFp8Row: 32 rows x 576 codes (18 KiB) per slot.  No widened copy of
//    the tile is made: every MFMA operand is read from the staging slot as
//    eight codes per lane and widened in registers (widen8, exact), QK's K
//    rows by plain 8-byte reads, PV's V^T by ds_read_b64_tr_b8 (below), so
//    the conversions overlap the matrix core instead of preceding it and
//    the LDS carries half the bytes.  The row's scale stays out of the
//    operands: it multiplies the row's summed logit and its softmax weight
//    before PV (the sum of the weights, the softmax denominator, is taken
//    unscaled).  LDS: the two slots and the S/P exchange buffer.
//  * kKvFp8Ds: 32 rows x 512 codes (16 KiB) per slot and the rows' four
//    block scales.  Once a tile has landed each wave widens the codes of
//    the dims it reads into one bf16 tile, laid out and swizzled as the
//    bf16 format's (wave 0 dims 0..287, wave 1 256..511; 256..287 are
//    written by both, with the same values, so the widened tile needs no
//    barrier of its own), each code as bf16(code x its block's scale), one
//    rounding, and QK / softmax / PV run on it as for bf16 rows.  The 64
//    rope dims are stored in bf16 already: they are gathered straight into
//    a rope buffer laid out as the bf16 tile's chunk group 8, one per ring
//    parity (the tile being computed keeps its rope while the next tile's
//    arrives), and wave 1's last four QK k-steps read them there.  LDS: the
//    codes part of the tile, 32 KiB, two 4-KiB rope buffers, two 16-KiB
//    slots.
constexpr int kF8TileB = kMlaRows * kDqk;   // 18432: one tile of per-token codes
constexpr int kDsTileB = kMlaRows * kDv;    // 16384: one tile of fp8_ds_mla codes
constexpr int kDsStageOff = kRopeOff + 2 * 4096;   // first staging slot (after the two rope buffers)
static_assert(2 * kF8TileB + 4096 <= 2 * kDmaTileB, "FP8 staging and exchange buffer fit the ring");
static_assert(kDsStageOff + 2 * kDsTileB <= 2 * kDmaTileB, "fp8_ds_mla staging fits the ring");

// With n_split > 1, workgroup (query, slice) covers one slice of the query's
// tiles (a contiguous range of 32-entry tiles) and leaves its unnormalised
// partial in `part` (O, the fixed exponent reference and the weight sum per
// head, the layout mla_merge_kernel reads); an empty slice leaves 0, -inf, 0.
template <bool OUT_F32, int KVF>
__global__ __launch_bounds__(kPairThreads, 1) void sparse_mla_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ kv, const float* __restrict__ kv_scale, int n_k,
    const int32_t* __restrict__ idx, int n_q, int K, float scale_log2, void* __restrict__ out,
    float* __restrict__ lse, int n_split, float* __restrict__ part) {
  constexpr bool FP8 = KVF != kKvBf16, ROW = KVF == kKvFp8Row, DS = KVF == kKvFp8Ds;
  // bf16: tiles 0 and 1; FP8: the bf16 tile (and rope buffers), then staging slots 0 and 1
  __shared__ __attribute__((aligned(1024))) uint8_t s_ring[2 * kDmaTileB];
  // per-row scales of the two staging slots: kKvFp8Row lane l's word (rows
  // l & 31), kKvFp8Ds four per row
  __shared__ __attribute__((aligned(16))) float s_sc[2][DS ? 4 * kMlaRows : 64];
  __shared__ __attribute__((aligned(1024))) uint8_t s_x[4096];
  __shared__ __attribute__((aligned(1024))) int s_idx[2][kIdxChunk];
  __shared__ float s_l[kHeads];
  __shared__ int s_red[2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int d = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qi = blockIdx.x / n_split, split = blockIdx.x % n_split;
  float* mypart = part ? part + (int64_t)blockIdx.x * kMlaPartFloats : nullptr;
  const int h = lane >> 5, c32 = lane & 31;
  const int32_t* irow = idx + (int64_t)qi * K;

  // ---- Q: block 0 = own heads 32d+c32, block 1 = partner heads; dims 288d +
  // 16ks + 8h .. +7.  Issued first: it does not depend on the extent, so its
  // loads and the extent loads below share one round trip ----
  bf16x8 qf[2][kPairKs];
#pragma unroll
  for (int hb = 0; hb < 2; ++hb) {
    const uint16_t* src = q + ((int64_t)qi * kHeads + 32 * (d ^ hb) + c32) * kDqk + 16 * kPairKs * d + 8 * h;
#pragma unroll
    for (int ks = 0; ks < kPairKs; ++ks) qf[hb][ks] = *reinterpret_cast<const bf16x8*>(src + 16 * ks);
  }

  // ---- extent of the selection: entries [0, n_ext) hold every valid index ----
  // The loads take clamped positions and are all issued before any is
  // tested, so they are in flight together.
  constexpr int kExtLoads = SMA_MAX_TOPK_DEV / kPairThreads;
  int ext[kExtLoads];
#pragma unroll
  for (int e = 0; e < kExtLoads; ++e) ext[e] = irow[min(e * kPairThreads + tid, K - 1)];
  int last = -1;
#pragma unroll
  for (int e = 0; e < kExtLoads; ++e) {
    const int j = e * kPairThreads + tid;
    if (j < K && ext[e] >= 0 && ext[e] < n_k) last = j;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o, 64));
  if (lane == 0) s_red[d] = last;
  __syncthreads();
  const int n_ext = max(s_red[0], s_red[1]) + 1;
  // this workgroup's tiles [t_beg, t_end)
  const int n_tiles_all = (n_ext + kMlaRows - 1) / kMlaRows;
  const int tps = (n_tiles_all + n_split - 1) / n_split;
  const int t_beg = min(n_tiles_all, split * tps), t_end = min(n_tiles_all, t_beg + tps);
  if (mypart && t_beg == t_end) {   // empty slice: zero partial, reference -inf
    wait_vmcnt<0>();                 // the Q loads retire before the wave ends
    for (int i = tid; i < kHeads * kDv / 4; i += kPairThreads)
      reinterpret_cast<f32x4*>(mypart)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (tid < kHeads) {
      mypart[kHeads * kDv + tid] = -INFINITY;
      mypart[kHeads * kDv + kHeads + tid] = 0.f;
    }
    return;
  }
  if (n_ext == 0) {
    wait_vmcnt<0>();
    for (int i = tid; i < kHeads * kDv / 4; i += kPairThreads) {
      if constexpr (OUT_F32) {
        reinterpret_cast<f32x4*>(static_cast<float*>(out) + (int64_t)qi * kHeads * kDv)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      } else {
        reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + (int64_t)qi * kHeads * kDv)[i] = u32x2{0u, 0u};
      }
    }
    if (lse && tid < kHeads) lse[(int64_t)qi * kHeads + tid] = -INFINITY;
    return;
  }

  // ---- gather: wave d fills blocks (rg, cg) for rg = 2d, 2d+1 and all 9
  // chunk groups; lane l fetches row 8rg + (l >> 3), chunk 8cg + ((l & 7) ^
  // swz(row)) ----
  const int rg_row = lane >> 3;
  // The entries are staged through LDS in chunks of 8 tiles (one chunk
  // ahead), so the per-tile index reads are LDS reads and the only
  // vector-memory operations in flight are the gathers and chunk loads.
  auto stage_chunk = [&](int c) {
    const uint32_t dst = (uint32_t)(uintptr_t)(lds_u8*)&s_idx[c & 1][kIdxChunk / 2 * d];
#pragma unroll
    for (int i = 0; i < kIdxChunk / 2 / 64; ++i) {
      const int v = c * kIdxChunk + kIdxChunk / 2 * d + 64 * i + lane;
      dma_load4(irow + min(v, K - 1), dst + 256 * i);
    }
  };
  auto entry_raw = [&](int e) -> int { return s_idx[(e / kIdxChunk) & 1][e % kIdxChunk]; };
  auto entry_ok = [&](int e, int x) -> bool { return e < n_ext && x >= 0 && x < n_k; };
  const int r_lo = 16 * d + rg_row, r_hi = r_lo + 8;   // rows of row groups 2d and 2d+1
  const int c_lo = 16 * ((lane & 7) ^ tile_swz(r_lo)), c_hi = 16 * ((lane & 7) ^ tile_swz(r_hi));
  // FP8 staging: load k (0..17) of a tile brings 16 bytes to each lane,
  // lane l: row l & 31, 16-byte chunk 2k + (l >> 5) of its 576 codes, at
  // staging byte 1024k + 16l; wave d issues loads 9d .. 9d + 8, so a lane
  // reads one index per tile and its nine chunks are 32 bytes apart.
  auto issue_f8 = [&](int t, int b) -> uint32_t {   // returns the tile's row mask
    const int e = t * kMlaRows + (lane & 31);
    const int raw = entry_raw(e);
    const bool ok = entry_ok(e, raw);
    const int row = ok ? raw : 0;
    const uint8_t* src = kv + (int64_t)row * kDqk + 16 * (18 * d + (lane >> 5));
    const uint32_t dst = (uint32_t)(uintptr_t)(lds_u8*)(s_ring + b * kF8TileB + 1024 * 9 * d);
#define SMA_F8_LOAD(k) dma_load16_at<32 * (k)>(src, dst + 1024 * (k));
    SMA_F8_LOAD(0) SMA_F8_LOAD(1) SMA_F8_LOAD(2) SMA_F8_LOAD(3) SMA_F8_LOAD(4)
    SMA_F8_LOAD(5) SMA_F8_LOAD(6) SMA_F8_LOAD(7) SMA_F8_LOAD(8)
#undef SMA_F8_LOAD
    if (d == 0) dma_load4(kv_scale + row, (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)&s_sc[b][0]);
    return (uint32_t)__ballot(ok);
  };
  // fp8_ds_mla: codes as issue_f8 with 512-code rows (loads k = 0..15, wave
  // d issues 8d .. 8d + 7), the 32 rows' scale chunks by wave 0's lanes 0..31
  // into s_sc, and the rope chunks of row groups 2d, 2d + 1 into the rope
  // buffer of parity b as the bf16 layout's blocks (rg, 8).
  auto issue_ds = [&](int t, int b) -> uint32_t {
    const int e = t * kMlaRows + (lane & 31);
    const int raw = entry_raw(e);
    const bool ok = entry_ok(e, raw);
    const uint8_t* rowp = kv + (int64_t)(ok ? raw : 0) * kDsRowB;
    const uint8_t* src = rowp + 256 * d + 16 * (lane >> 5);
    const uint32_t dst = (uint32_t)(uintptr_t)(lds_u8*)(s_ring + kDsStageOff + b * kDsTileB + 8192 * d);
#define SMA_DS_LOAD(k) dma_load16_at<32 * (k)>(src, dst + 1024 * (k));
    SMA_DS_LOAD(0) SMA_DS_LOAD(1) SMA_DS_LOAD(2) SMA_DS_LOAD(3)
    SMA_DS_LOAD(4) SMA_DS_LOAD(5) SMA_DS_LOAD(6) SMA_DS_LOAD(7)
#undef SMA_DS_LOAD
    if (d == 0 && lane < 32)
      dma_load16(rowp + kDsScaleOff, (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)&s_sc[b][0]);
    const int raw_lo = entry_raw(t * kMlaRows + r_lo), raw_hi = entry_raw(t * kMlaRows + r_hi);
    const bool ok_lo = entry_ok(t * kMlaRows + r_lo, raw_lo), ok_hi = entry_ok(t * kMlaRows + r_hi, raw_hi);
    const uint32_t rdst = (uint32_t)(uintptr_t)(lds_u8*)(s_ring + kRopeOff + 4096 * b + 1024 * 2 * d);
    dma_load16(kv + (int64_t)(ok_lo ? raw_lo : 0) * kDsRowB + kDsRopeOff + c_lo, rdst);
    dma_load16(kv + (int64_t)(ok_hi ? raw_hi : 0) * kDsRowB + kDsRopeOff + c_hi, rdst + 1024);
    return (uint32_t)__ballot(ok);
  };
  auto issue_tile = [&](int t, int b) -> uint32_t {   // returns the tile's row mask
    if constexpr (DS) return issue_ds(t, b);
    if constexpr (ROW) return issue_f8(t, b);
    const int raw_lo = entry_raw(t * kMlaRows + r_lo), raw_hi = entry_raw(t * kMlaRows + r_hi);
    const bool ok_lo = entry_ok(t * kMlaRows + r_lo, raw_lo), ok_hi = entry_ok(t * kMlaRows + r_hi, raw_hi);
    const uint8_t* src_lo = kv + (int64_t)(ok_lo ? raw_lo : 0) * kDmaRowB + c_lo;
    const uint8_t* src_hi = kv + (int64_t)(ok_hi ? raw_hi : 0) * kDmaRowB + c_hi;
    const uint32_t dst = (uint32_t)(uintptr_t)(lds_u8*)(s_ring + b * kDmaTileB + tile_block(2 * d, 0));
    // chunk group cg of both rows: global offset 128 cg, LDS block (rg, cg)
#define SMA_TILE_CG(cg)                                           \
  dma_load16_at<128 * (cg)>(src_lo, dst + 4096 * (cg));           \
  dma_load16_at<128 * (cg)>(src_hi, dst + 4096 * (cg) + 1024);
    SMA_TILE_CG(0) SMA_TILE_CG(1) SMA_TILE_CG(2) SMA_TILE_CG(3) SMA_TILE_CG(4)
    SMA_TILE_CG(5) SMA_TILE_CG(6) SMA_TILE_CG(7) SMA_TILE_CG(8)
#undef SMA_TILE_CG
    static_assert(kDmaRowB / 128 == 9, "nine chunk groups per row");
    // row mask of the whole tile: lane r (< 32) checks row r
    const int e_m = t * kMlaRows + (lane & 31);
    return (uint32_t)__ballot(entry_ok(e_m, entry_raw(e_m)));
  };
  // Retire the Q and extent loads: from here on the wave's outstanding
  // vector-memory operations are gathers and index-chunk loads only.
  wait_vmcnt<0>();

  // K operand of k-step ks (global 18d+ks): row c32, chunk c = 36d + 2ks + h;
  // for ks = 4j + p the chunk group is that of 36d + 2p + h plus j and the
  // slot that of 36d + 2p + h, so four bases and immediate offsets 4096j.
  int kb[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int c = 36 * d + 2 * p + h;
    kb[p] = tile_block(c32 >> 3, c >> 3) + 128 * (c32 & 7) + 16 * ((c & 7) ^ tile_swz(c32));
  }
  // V^T operand of M-tile m (dims 256d+32m..), k-step kk, half e: 16-lane group b = lane>>4
  // reads row 16kk + 8e + 4h + (L>>2) at dims 256d + 32m + 16(b&1) + 4(L&3), L = lane&15;
  // chunk group 4d + (m>>1), slot from 4(m&1) + 2(b&1) + ((L&3)>>1): four bases
  // (e, m&1) and immediate offsets 4096(m>>1) + 2048kk.
  const int L = lane & 15;
  int vb[2][2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int m1 = 0; m1 < 2; ++m1) {
      const int r = 8 * e + 4 * h + (L >> 2);
      const int c7 = 4 * m1 + 2 * ((lane >> 4) & 1) + ((L & 3) >> 1);
      vb[e][m1] = tile_block(e, 4 * d) + 128 * (r & 7) + 16 * (c7 ^ tile_swz(r)) + 8 * (L & 1);
    }

  // Per-token FP8 rows are read from their staging slot and widened operand
  // by operand in registers.  QK's A operand (row c32, dims 288d + 16ks +
  // 8h .. +7) is eight bytes of piece 18d + ks of the row: staging byte
  // 9216d + 16 c32 + 8h plus 1024 (ks >> 1) + 512 (ks & 1).  PV's V^T
  // operand comes from ds_read_b64_tr_b8: in a 16-lane group G, output lane
  // 16G + 8p + i takes byte i of the eight-byte reads of lanes 16G + 2e + p,
  // e = 0..7, as its elements e.  So lane s = 16G + 2e + p reads row
  // 16kk + 8(e >> 2) + 4(G >> 1) + (e & 3) (the key order of P's registers,
  // as the bf16 reads) at dims 256d + 32m + 16(G & 1) + 8p .. +7: staging
  // byte 8192d + 512(G & 1) + 16 row + 8p plus 1024m + 256kk.
  const int kb8 = 9216 * d + 16 * c32 + 8 * h;
  int vb8;
  {
    const int G = lane >> 4, e = (lane & 15) >> 1, p = lane & 1;
    vb8 = 8192 * d + 512 * (G & 1) + 16 * (8 * (e >> 2) + 4 * (G >> 1) + (e & 3)) + 8 * p;
  }

  f32x16v o[kPairMt][2];
  float m_ref = -INFINITY, m_max = -INFINITY, l_run = 0.f;

  // One sweep over the entries with a FIXED per-head exponent reference
  // (the first tile's maximum, or the exact maximum on a rerun).  Returns
  // whether some logit passed m_ref + kRefGap.
  auto sweep = [&]() -> bool {
#pragma unroll
    for (int m = 0; m < kPairMt; ++m) o[m][0] = o[m][1] = f32x16v{};
    l_run = 0.f;
    bool far = false;
    // Vector-memory operations of iteration t: [index chunk], gather(t+1).
    // Chunk c (entries 256c ..) sits in slot c & 1.  The slice's first chunk
    // and the one after it are staged before the loop; later, chunk k + 1 is
    // staged at tile 8k, seven tiles before its first entries are read (the
    // issue of tile 8k + 8 at iteration 8k + 7), when chunk k - 1 is dead.
    constexpr int kTpc = kIdxChunk / kMlaRows;   // tiles per index chunk
    const int c_beg = t_beg / kTpc;
    stage_chunk(c_beg);
    if ((c_beg + 1) * kTpc < t_end) stage_chunk(c_beg + 1);
    wait_vmcnt<0>();
    block_sync_lds();
    uint32_t mask = issue_tile(t_beg, t_beg & 1);
    for (int t = t_beg; t < t_end; ++t) {
      wait_vmcnt<0>();     // tile t (and any index chunk) has landed
      block_sync_lds();    // for both waves; tile t-1's slot and the exchange buffers are free
      if (t > t_beg && t % kTpc == 0 && (t / kTpc + 1) * kTpc < t_end) stage_chunk(t / kTpc + 1);
      uint32_t mask_next = 0;
      if (t + 1 < t_end) mask_next = issue_tile(t + 1, (t + 1) & 1);
      // bf16: tile t's ring slot; per-token FP8: its staging slot;
      // fp8_ds_mla: the widened tile
      uint8_t* tile = ROW ? s_ring + (t & 1) * kF8TileB : DS ? s_ring : s_ring + (t & 1) * kDmaTileB;
      // fp8_ds_mla: tile t's rope dims sit in the rope buffer of its parity
      const int rope_add = DS ? 4096 * (t & 1) : 0;
      if constexpr (DS) {
        const uint8_t* stage = s_ring + kDsStageOff + (t & 1) * kDsTileB;
        const f32x4 bsc = *reinterpret_cast<const f32x4*>(&s_sc[t & 1][4 * (lane & 31)]);
        if (d == 0) widen_ds_dims<0, 9>(stage, tile, lane, bsc);
        else widen_ds_dims<16, 8>(stage, tile, lane, bsc);
      }

      // ---- partial S^T over this wave's dims, both head blocks ----
      constexpr int kPf = 3;
      // (wave 1's k-steps 14..17 are the rope dims, chunk group 8; wave 0's
      // are code dims)
      const int rope_k = d ? rope_add : 0;
      auto kread = [&](int ks) -> bf16x8 {
        if constexpr (ROW) {
          const u32x2 c = *reinterpret_cast<const u32x2*>(tile + kb8 + 1024 * (ks >> 1) + 512 * (ks & 1));
          return widen8(c[0], c[1]);
        } else {
          const int ra = ks >= kPairKs - 4 ? rope_k : 0;
          return *reinterpret_cast<const bf16x8*>(tile + kb[ks & 3] + (ks >> 2) * 4096 + ra);
        }
      };
      f32x16v s_own, s_oth;
      bf16x8 kop[kPf];
#pragma unroll
      for (int ks = 0; ks < kPf; ++ks) kop[ks] = kread(ks);
#pragma unroll
      for (int ks = 0; ks < kPairKs - 2; ++ks) {
        const bf16x8 a = kop[ks % kPf];
        if (ks + kPf < kPairKs) kop[ks % kPf] = kread(ks + kPf);
        if (ks == 0) {
          mfma32_vgpr_first(s_oth, a, qf[1][0]);
          mfma32_vgpr_first(s_own, a, qf[0][0]);
        } else {
          mfma32_vgpr(s_oth, a, qf[1][ks]);
          mfma32_vgpr(s_own, a, qf[0][ks]);
        }
      }
      // The partner's block finishes first, so its half-sum goes out while
      // the last own-block MFMAs run.
      constexpr int kA = kPairKs - 2, kB = kPairKs - 1;
      mfma32_vgpr(s_oth, kop[kA % kPf], qf[1][kA]);
      mfma32_vgpr(s_oth, kop[kB % kPf], qf[1][kB]);
      mfma32_vgpr(s_own, kop[kA % kPf], qf[0][kA]);
      mfma32_vgpr_drain1(s_oth);

      // ---- exchange half-sums: wave 1 writes into the (now dead) rope blocks, wave 0 into s_x ----
      // (per-token FP8: a buffer of its own past the two staging slots)
      uint8_t* xa = ROW ? s_ring + 2 * kF8TileB : tile + kRopeOff + rope_add;
      uint8_t* xw = d ? xa : s_x;   // written by this wave
      uint8_t* xr = d ? s_x : xa;   // written by the partner
#pragma unroll
      for (int p = 0; p < 4; ++p)
        *reinterpret_cast<f32x4*>(xw + 1024 * p + 16 * lane) =
            f32x4{s_oth[4 * p], s_oth[4 * p + 1], s_oth[4 * p + 2], s_oth[4 * p + 3]};
      mfma32_vgpr(s_own, kop[kB % kPf], qf[0][kB]);
      block_sync_lds();
      f32x4 y[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) y[p] = *reinterpret_cast<const f32x4*>(xr + 1024 * p + 16 * lane);
      mfma32_vgpr_drain(s_own, s_oth);
#pragma unroll
      for (int p = 0; p < 4; ++p)
#pragma unroll
        for (int r = 0; r < 4; ++r) s_own[4 * p + r] += y[p][r];
      if constexpr (ROW) {   // the rows' scales on their summed logits (rows 8p + 4h + r)
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const f32x4 rs = *reinterpret_cast<const f32x4*>(&s_sc[t & 1][8 * p + 4 * h]);
#pragma unroll
          for (int r = 0; r < 4; ++r) s_own[4 * p + r] *= rs[r];
        }
      }

      // ---- softmax weights of the own heads: element j is row 8(j>>2) + 4h + (j&3) ----
      // A full tile (every row valid; the mask is the same in every lane)
      // needs no masking.  Weights are 2^(s tau log2e - m_ref); scale_log2 > 0,
      // so the row maximum is taken on the raw sums.  No clamp is needed: a
      // weight can only exceed 2^kRefGap when `far` is set, and then the
      // sweep's results are discarded.
      const bool full = mask == 0xFFFFFFFFu;
      bf16x8 pb[2];
      float ps = 0.f;
      auto softmax = [&](auto masked) {
        constexpr bool M = decltype(masked)::value;
        const uint32_t mh = mask >> (4 * h);
        auto row_ok = [&](int j) { return ((mh >> (8 * (j >> 2) + (j & 3))) & 1u) != 0u; };
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, !M || row_ok(j) ? s_own[j] : -INFINITY);
        mx *= scale_log2;
        {   // lanes l and l ^ 32 hold the same head: v_permlane32_swap hands each the other's value
          const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
          mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        if (m_ref == -INFINITY) m_ref = mx;   // first tile holding a valid row
        m_max = fmaxf(m_max, mx);
        far |= mx > m_ref + kRefGap;
        const float neg_ref = -m_ref;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s_own[j], scale_log2, neg_ref));
          if constexpr (M) pe = row_ok(j) ? pe : 0.f;
          ps += pe;
          if constexpr (ROW)   // PV takes the codes: the row's scale goes on its weight
            pb[j >> 3][j & 7] = (__bf16)(pe * s_sc[t & 1][8 * (j >> 2) + 4 * h + (j & 3)]);
          else
            pb[j >> 3][j & 7] = (__bf16)pe;
        }
      };
      // `full` is the same in every lane: one uniform branch keeps the row
      // masking out of the (common) full tiles' code
      if (full) softmax(std::false_type{});
      else softmax(std::true_type{});
      l_run += ps;

      // ---- P to the partner (into the buffer just read), P of the partner's heads back ----
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) *reinterpret_cast<bf16x8*>(xr + 1024 * kk + 16 * lane) = pb[kk];
      block_sync_lds();
      bf16x8 pq[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) pq[kk] = *reinterpret_cast<const bf16x8*>(xw + 1024 * kk + 16 * lane);

      // ---- O^T += V^T . P^T over this wave's dims, both head blocks ----
      auto vread = [&](int m, int kk) -> bf16x8 {
        if constexpr (ROW) {
          const i32x2v c = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(tile + vb8 + 1024 * m + 256 * kk));
          return widen8((uint32_t)c[0], (uint32_t)c[1]);
        }
        const int off = 4096 * (m >> 1) + 2048 * kk;
        const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + vb[0][m & 1] + off));
        const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + vb[1][m & 1] + off));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8 vop[2][2];
      vop[0][0] = vread(0, 0);
      vop[0][1] = vread(0, 1);
#pragma unroll
      for (int m = 0; m < kPairMt; ++m) {
        if (m + 1 < kPairMt) {
          vop[(m + 1) & 1][0] = vread(m + 1, 0);
          vop[(m + 1) & 1][1] = vread(m + 1, 1);
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          o[m][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[m & 1][kk], pb[kk], o[m][0], 0, 0, 0);
          o[m][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[m & 1][kk], pq[kk], o[m][1], 0, 0, 0);
        }
      }
      mask = mask_next;
    }
    return far;
  };

  // Fast sweep; a query whose logits rose more than 2^kRefGap above its first
  // valid tile's maximum is swept again with the exact maximum as the
  // reference (one copy of the sweep code, run at most twice).
#pragma nounroll
  for (int pass = 0; pass < 2; ++pass) {
    const bool far = __ballot(sweep()) != 0;
    block_sync_lds();   // both waves are done with the ring and s_x
    if (lane == 0) s_red[d] = far ? 1 : 0;
    block_sync_lds();
    const bool redo = (s_red[0] | s_red[1]) != 0;
    block_sync_lds();   // flags read before they are rewritten
    if (!redo) break;
    m_ref = m_max;      // this lane's head, over every valid row
  }

  // ---- normalise and write: o[m][hb] holds head 32(d^hb)+c32, dims 256d + 32m + 8jj + 4h + r ----
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (mypart) {   // the slice's partial: unnormalised O, reference (log2 units), weight sum
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      float* prow = mypart + (32 * (d ^ hb) + c32) * kDv + 256 * d + 4 * h;
#pragma unroll
      for (int m = 0; m < kPairMt; ++m)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *reinterpret_cast<f32x4*>(prow + 32 * m + 8 * jj) =
              f32x4{o[m][hb][4 * jj], o[m][hb][4 * jj + 1], o[m][hb][4 * jj + 2], o[m][hb][4 * jj + 3]};
    }
    if (h == 0) {
      mypart[kHeads * kDv + 32 * d + c32] = m_ref;
      mypart[kHeads * kDv + kHeads + 32 * d + c32] = l_tot;
    }
    return;
  }
  if (h == 0) s_l[32 * d + c32] = l_tot;
  block_sync_lds();
  const float inv[2] = {1.f / l_tot, 1.f / s_l[32 * (d ^ 1) + c32]};
  if constexpr (OUT_F32) {
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int64_t row_off = ((int64_t)qi * kHeads + 32 * (d ^ hb) + c32) * kDv + 256 * d + 4 * h;
#pragma unroll
      for (int m = 0; m < kPairMt; ++m)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 r = f32x4{o[m][hb][4 * jj], o[m][hb][4 * jj + 1], o[m][hb][4 * jj + 2], o[m][hb][4 * jj + 3]} *
                          inv[hb];
          *reinterpret_cast<f32x4*>(static_cast<float*>(out) + row_off + 32 * m + 8 * jj) = r;
        }
    }
  } else {
    // The query's bf16 output [64 heads][512 dims] is one contiguous 64 KiB
    // block: stage it in the (now idle) tile ring as rows of 1 KiB whose
    // 16-byte chunk c sits at slot c ^ (head & 63), then write it with
    // 16-byte stores by consecutive lanes.  Lanes of one accumulator store
    // hold 32 heads, which the slot rotation spreads over the banks.
    uint8_t* obuf = s_ring;
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int head = 32 * (d ^ hb) + c32;
      uint8_t* orow = obuf + head * 1024 + 8 * h;
#pragma unroll
      for (int m = 0; m < kPairMt; ++m)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const f32x4 r = f32x4{o[m][hb][4 * jj], o[m][hb][4 * jj + 1], o[m][hb][4 * jj + 2], o[m][hb][4 * jj + 3]} *
                          inv[hb];
          const int chunk = 32 * d + 4 * m + jj;   // dims 8 chunk .. 8 chunk + 7
          *reinterpret_cast<u32x2*>(orow + 16 * (chunk ^ (head & 63))) =
              u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
        }
    }
    block_sync_lds();
    uint8_t* og = reinterpret_cast<uint8_t*>(out) + (int64_t)qi * kHeads * kDv * 2;
#pragma unroll 8
    for (int i = 0; i < kHeads * kDv * 2 / 16 / kPairThreads; ++i) {
      const int c = tid + kPairThreads * i, head = c >> 6, cc = c & 63;
      *reinterpret_cast<u32x4*>(og + 16 * c) = *reinterpret_cast<const u32x4*>(obuf + head * 1024 + 16 * (cc ^ (head & 63)));
    }
  }
  if (lse && h == 0) lse[(int64_t)qi * kHeads + 32 * d + c32] = (m_ref + __log2f(l_tot)) * 0.69314718055994531f;
}

int mla_split_count(int n_q, int top_k) {
  if (n_q <= 0) return 1;
  const int cus = device_cu_count();
  if (n_q >= cus) return 1;
  int s = (2 * cus + n_q - 1) / n_q;            // about two workgroups per CU
  s = std::min(s, std::min(16, std::max(1, top_k / 128)));   // slices of at least 128 rows
  return std::max(1, s);
}

size_t mla_split_bytes(int n_q, int n_split) {
  return n_split > 1 ? (size_t)n_q * n_split * kMlaPartFloats * sizeof(float) : 0;
}

hipError_t launch_sparse_mla(const MlaArgs& A, hipStream_t st) {
  if (A.n_q <= 0) return hipSuccess;
  const float scale_log2 = A.sm_scale * 1.4426950408889634f;
  const dim3 block(kPairThreads);
  const uint8_t* kv8 = static_cast<const uint8_t*>(A.kv);
  // small batches split each query's rows across workgroups, into as many
  // slices as the workspace holds partials for (up to the preferred count)
  int n_split = mla_split_count(A.n_q, A.top_k);
  if (n_split > 1) {
    const size_t per_slice = mla_split_bytes(A.n_q, 2) / 2;
    const size_t fit = A.ws ? A.ws_bytes / per_slice : 0;
    if ((size_t)n_split > fit) n_split = (int)fit;
    if (n_split < 2) n_split = 1;
  }
  float* part = n_split > 1 ? static_cast<float*>(A.ws) : nullptr;
  const dim3 grid_s((unsigned)(A.n_q * n_split));
#define SMA_MLA_LAUNCH(F32, KVF)                                                                              \
  hipLaunchKernelGGL((sparse_mla_kernel<F32, KVF>), grid_s, block, 0, st, A.q, kv8, A.kv_scale, (int)A.n_k, A.idx, \
                     A.n_q, A.top_k, scale_log2, A.out, A.lse, n_split, part)
  if (A.fp8 && A.ds_mla) {
    if (A.out_f32) SMA_MLA_LAUNCH(true, kKvFp8Ds);
    else SMA_MLA_LAUNCH(false, kKvFp8Ds);
  } else if (A.fp8) {
    if (A.out_f32) SMA_MLA_LAUNCH(true, kKvFp8Row);
    else SMA_MLA_LAUNCH(false, kKvFp8Row);
  } else {
    if (A.out_f32) SMA_MLA_LAUNCH(true, kKvBf16);
    else SMA_MLA_LAUNCH(false, kKvBf16);
  }
#undef SMA_MLA_LAUNCH
  if (n_split > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid_m((unsigned)A.n_q, kHeads / kMergeHeads);
    if (A.out_f32)
      hipLaunchKernelGGL((mla_merge_kernel<true>), grid_m, dim3(256), 0, st, part, n_split, A.out, A.lse);
    else
      hipLaunchKernelGGL((mla_merge_kernel<false>), grid_m, dim3(256), 0, st, part, n_split, A.out, A.lse);
  }
  return hipGetLastError();
}

}  // namespace sma
