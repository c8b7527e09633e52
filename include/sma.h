/*
 * sma.h — C ABI of the MI355X (gfx950) sparse-MLA prefill path:
 *   indexer scores -> per-query top-k -> sparse MLA over the selected
 *   latent rows, plus one PCP rank's load-balanced share.
 *
 * The operations follow the GLM-5.3 part 2 article (PCP, DCP and Hybrid
 * HiSparse on 16 H200):
 *   - section "Pourquoi pas TP ou DP ?": an indexer scores every earlier
 *     token of the prompt and keeps the 2,048 that sparse MLA consults;
 *   - section "PCP : répartir les tokens, pas les têtes": one latent KV row
 *     serves all 64 heads; a prompt is cut into 16 chunks and each of 8
 *     ranks computes one early and one late chunk;
 *   - footnote 1: QK over 576 dims, PV over 512, a 4-byte index per
 *     selected row, bf16 query and output;
 *   - footnote 3: an FP8 key row carries a 4-byte scale.
 * The indexer's form (ReLU of per-head dot products, weighted by a per-head
 * weight and summed over heads, causal with the query's own token
 * included), the lowest-position tie-break and "value = first 512 dims"
 * are the readings this library implements where the pages are silent.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is DEVICE memory owned by the caller, row-major,
 *    contiguous except where a stride argument is given.  The library never
 *    allocates, frees or keeps a pointer after returning.  Scratch memory is
 *    the caller's workspace (sma_workspace_bytes).
 *  - bf16 tensors are passed as uint16_t bit patterns.  FP8 tensors are OCP
 *    e4m3fn codes (uint8_t) with one fp32 scale per row (value = code*scale,
 *    scale >= 0).
 *  - `stream` is a hipStream_t (NULL = the null stream).  All work is
 *    enqueued on it in order; no call synchronises the host.
 *  - Arguments are validated on the host before anything is launched.  A bad
 *    call returns a negative sma_status, launches nothing, and leaves a
 *    message for sma_last_error() (thread-local).  A failed launch returns
 *    SMA_ERR_HIP.  Faults inside kernels surface at the caller's next
 *    synchronisation.
 *  - Device-resident values the host cannot see are made safe in the
 *    kernels: a query position p is clamped to [-1, n_k-1] (p = -1 means an
 *    empty causal prefix); an index outside [0, n_k) in an index list is
 *    skipped like the -1 padding.
 *  - Debug build (libsma_debug.so; sma_build_flags() has
 *    SMA_BUILD_DEBUG_CHECKS): the same entry points, which also scan each
 *    device-resident index list and position array before the launch that
 *    reads it and return SMA_ERR_INVALID_ARG, with nothing else launched,
 *    for a value the release build would skip or clamp (a position outside
 *    [-1, n_k-1]; an index list entry below -1 or, except in a DCP shard's
 *    global list, at or past n_k); and fill the workspace (or the static
 *    scratch) with 0xFF bytes, fp32 NaN, before using it.  These checks
 *    synchronise the stream and are meant for testing, not for capture.
 *  - Results are deterministic: the same inputs give bit-identical outputs,
 *    whatever the launch split (a PCP share equals the matching rows of the
 *    unsharded call).
 *  - Only gfx950 devices are supported (SMA_ERR_UNSUPPORTED otherwise).
 */
#ifndef SMA_H
#define SMA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SMA_OK = 0,
  SMA_ERR_INVALID_ARG = -1,
  SMA_ERR_UNSUPPORTED = -2,
  SMA_ERR_WORKSPACE = -3,
  SMA_ERR_HIP = -4
} sma_status;

/* SMA_DT_FP8_DS_MLA: FlashMLA's 656-byte fp8_ds_mla latent row (GLM-5.3
 * part 2, footnote 1, names it and gives its 656 bytes; the internal layout
 * is not on the page and is taken from FlashMLA's public description): bytes
 * 0..511 the e4m3fn codes of latent dims 0..511, bytes 512..527 four fp32
 * scales (scale b for dims 128b .. 128b+127), bytes 528..655 rope dims
 * 512..575 as bf16.  Accepted as the KV of the sparse-MLA entry points
 * (kv_scale must then be NULL); rows are 656 bytes apart. */
typedef enum { SMA_DT_BF16 = 0, SMA_DT_FP8_E4M3 = 1, SMA_DT_FP32 = 2, SMA_DT_FP8_DS_MLA = 3 } sma_dtype;

typedef enum {
  SMA_OP_INDEX_SCORES = 0,
  SMA_OP_TOPK = 1,
  SMA_OP_SPARSE_MLA = 2,
  SMA_OP_PREFILL = 3,
  SMA_OP_PCP_SHARE = 4,
  SMA_OP_DCP_PARTIAL = 5,
  SMA_OP_DENSE_MHA = 6
} sma_op;

/* Fixed MLA geometry: 64 heads share one 576-wide latent row (512 latent +
 * 64 rope); the value is the first 512 dims. */
#define SMA_HEADS 64
#define SMA_D_QK 576
#define SMA_D_V 512
#define SMA_MAX_TOPK 2048

/*
 * sma_index_scores — indexer scores over each query's causal prefix
 * (GLM-5.3 part 2, "Pourquoi pas TP ou DP ?").
 *
 *   scores[i*ld + s] = sum_h w[i*w_stride + h] * max(0, q_idx[i,h,:] . k_idx[s,:])
 *   for 0 <= s <= p_i, p_i = clamp(q_pos[i], -1, n_k-1);
 *   with FP8 keys the key row is code*k_scale[s].
 *
 *  q_idx    [n_q, h_idx, d_idx] bf16
 *  w        fp32, element (i,h) at w[i*w_stride + h]; w_stride = 0 shares
 *           one [h_idx] vector across queries
 *  k_idx    [n_k, d_idx] bf16, or e4m3fn codes when k_dtype = SMA_DT_FP8_E4M3
 *  k_scale  [n_k] fp32 when FP8, else must be NULL
 *  q_pos    [n_q] int32 global positions
 *  scores   [n_q, ld_scores] fp32; only s <= p_i is written, the rest of the
 *           row is left untouched
 *  Supported: h_idx in {8,16,32,64}, d_idx in {64,128}, ld_scores >= n_k,
 *  n_k < 2^31.  n_q = 0 is a no-op.  Products are bf16 x bf16 with fp32
 *  accumulation; the ReLU, head weights and head sum are fp32.
 */
sma_status sma_index_scores(const uint16_t* q_idx, const float* w, int64_t w_stride,
                            const void* k_idx, const float* k_scale, int32_t k_dtype,
                            const int32_t* q_pos, int32_t n_q, int64_t n_k,
                            int32_t h_idx, int32_t d_idx,
                            float* scores, int64_t ld_scores, void* stream);

/*
 * sma_quantize_fp8_rows — per-row FP8 quantisation of bf16 rows, the way the
 * FP8 indexer's operands are stored: one fp32 scale per row of d values
 * (DeepSeek multi-node page, "Quantification": activation scales over
 * 128-element vectors; GLM-5.3 part 2, footnote 3: a key row is 128 FP8
 * values plus a 4-byte scale).
 *
 *   scale[r]   = amax_j |x[r,j]| / 448                       (fp32, rounded)
 *   codes[r,j] = e4m3fn(clamp(x[r,j] / scale[r], -448, 448)) (fp32 division,
 *                nearest-even code); a row of zeros gets scale 0, codes 0
 *
 *  x      [n_rows, d] bf16, 16-byte aligned; inputs must be finite
 *  codes  [n_rows, d] uint8, 8-byte aligned;  scale [n_rows] fp32
 *  Supported: d in {64, 128}, 0 <= n_rows <= 2^36.  A query's 64 head rows
 *  of q_I are 64 rows here (scale index i*64 + h).
 */
sma_status sma_quantize_fp8_rows(const uint16_t* x, int64_t n_rows, int32_t d, uint8_t* codes, float* scale,
                                 void* stream);

/*
 * sma_index_scores_fp8 — the indexer scores of sma_index_scores with FP8
 * queries and FP8 keys (footnote 3 of the same article stores the keys so;
 * the queries carry one scale per head row, as sma_quantize_fp8_rows makes
 * them):
 *
 *   scores[i*ld + s] = sum_h w[i*w_stride + h]
 *                      * max(0, (q_scale[i*64+h] * e4m3(q_idx[i,h,:]))
 *                               . (k_scale[s] * e4m3(k_idx[s,:])))
 *
 *  q_idx [n_q, 64, 128] e4m3fn codes (16-byte aligned), q_scale [n_q, 64]
 *  fp32 >= 0; k_idx [n_k, 128] codes, k_scale [n_k] fp32 >= 0; the rest as
 *  sma_index_scores.  The dot products run on e4m3 x e4m3 MFMA with fp32
 *  accumulation (exact products); the scales, ReLU, head weights and head
 *  sum are fp32.
 *  Supported: h_idx = 64, d_idx = 128 only (SMA_ERR_UNSUPPORTED otherwise).
 */
sma_status sma_index_scores_fp8(const uint8_t* q_idx, const float* q_scale, const float* w, int64_t w_stride,
                                const uint8_t* k_idx, const float* k_scale, const int32_t* q_pos, int32_t n_q,
                                int64_t n_k, int32_t h_idx, int32_t d_idx, float* scores, int64_t ld_scores,
                                void* stream);

/*
 * sma_topk_select — per-query top-k of the causal scores (same article,
 * "Pourquoi pas TP ou DP ?"; 4-byte indices, footnote 1).
 *
 *  Row i holds n_i = clamp(q_pos[i], -1, n_k-1) + 1 scores at
 *  scores[i*ld_scores + 0 .. n_i-1].  idx[i*top_k + 0 .. m_i-1] receives the
 *  m_i = min(top_k, n_i) positions with the largest scores, in ascending
 *  position order; slots m_i .. top_k-1 receive -1.  Ties at the threshold
 *  go to the lowest positions; -0.0 and +0.0 are one value; a NaN (either
 *  sign, any payload) ranks below every number, -inf included, so NaN
 *  positions are selected only when a row holds fewer than m_i numbers, the
 *  lowest NaN positions first.  Every row length and alignment follows this
 *  one rule.
 *  Supported: 1 <= top_k <= 2048, ld_scores >= n_k, n_k < 2^31.
 *  ws/ws_bytes: workspace (sma_workspace_bytes(SMA_OP_TOPK, ...), may be 0).
 */
sma_status sma_topk_select(const float* scores, int64_t ld_scores, const int32_t* q_pos,
                           int32_t n_q, int64_t n_k, int32_t top_k, int32_t* idx,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * sma_sparse_mla_prefill — absorbed ("MQA" mode) sparse MLA: all 64 heads
 * of query i attend over the latent rows idx[i, :] (same article, "PCP :
 * répartir les tokens, pas les têtes", "Essayez-le", footnote 1).
 *
 *   z_s      = sm_scale * q[i,h,:] . kv[s, 0:576]          for s in S_i
 *   out[i,h] = sum_s softmax(z)_s * kv[s, 0:512]
 *   lse[i,h] = log(sum_s exp(z_s))                          (natural log)
 *
 *  q        [n_q, 64, 576] bf16
 *  kv       [n_k, 576] bf16, or e4m3fn codes with kv_scale [n_k] fp32, or
 *           [n_k] 656-byte fp8_ds_mla rows (kv_dtype SMA_DT_FP8_DS_MLA,
 *           kv_scale NULL)
 *  idx      [n_q, top_k] int32; entries < 0 or >= n_k are skipped
 *  out      [n_q, 64, 512], out_dtype SMA_DT_BF16 or SMA_DT_FP32
 *  lse      [n_q, 64] fp32, or NULL.  A query with no valid index gets
 *           out = 0 and lse = -inf.
 *  Softmax and accumulation are fp32; QK and PV run on bf16 MFMA (an FP8
 *  row is widened to bf16 exactly and its scale multiplies the logit and
 *  the softmax weight; an fp8_ds_mla row's codes are widened as bf16(code x
 *  the scale of their 128-dim block), one rounding each, its rope dims
 *  taken as stored).
 *  sm_scale must be finite and > 0 (SMA_ERR_INVALID_ARG otherwise).
 *  Supported: 1 <= top_k <= 2048.  ws may be NULL (ws_bytes 0).  With a
 *  workspace (256-byte aligned), a batch of fewer queries than the device
 *  has compute units splits each query's rows into slices whose partial
 *  results are merged by log-sum-exp: with
 *  sma_workspace_bytes(SMA_OP_SPARSE_MLA, ...) bytes into the preferred
 *  number of slices, with less into as many as the workspace holds
 *  partials for.  Slices change the result only by rounding: fp32
 *  summation order, and the bf16 rounding of the softmax weights, which each
 *  slice takes against its own running maximum.
 */
sma_status sma_sparse_mla_prefill(const uint16_t* q, const void* kv, const float* kv_scale,
                                  int32_t kv_dtype, int64_t n_k, const int32_t* idx,
                                  int32_t n_q, int32_t top_k, float sm_scale,
                                  void* out, int32_t out_dtype, float* lse,
                                  void* ws, size_t ws_bytes, void* stream);

/*
 * sma_prefill — indexer -> top-k -> sparse MLA for n_q query rows at
 * positions q_pos against the n_k-row context.  Arguments as above.
 *  idx_out  [n_q, top_k] int32 or NULL (then kept in the workspace).
 *  The scores are produced block by block in the workspace; a larger
 *  workspace allows larger query blocks (fewer launches), never different
 *  results.  Minimum size: sma_workspace_bytes(SMA_OP_PREFILL, ...), which
 *  holds the index list and a block of min(n_q, 64) rows, for any n_q.
 */
sma_status sma_prefill(const uint16_t* q_idx, const float* w, int64_t w_stride,
                       const void* k_idx, const float* k_scale, int32_t k_dtype,
                       const uint16_t* q, const void* kv, const float* kv_scale, int32_t kv_dtype,
                       const int32_t* q_pos, int32_t n_q, int64_t n_k,
                       int32_t h_idx, int32_t d_idx, int32_t top_k, float sm_scale,
                       void* out, int32_t out_dtype, float* lse, int32_t* idx_out,
                       void* ws, size_t ws_bytes, void* stream);

/*
 * sma_prefill_fp8_indexer — sma_prefill with the indexer of
 * sma_index_scores_fp8 (FP8 queries and keys, h_idx = 64, d_idx = 128);
 * top-k and sparse MLA as in sma_prefill, the same workspace
 * (sma_workspace_bytes(SMA_OP_PREFILL, ...)).
 */
sma_status sma_prefill_fp8_indexer(const uint8_t* q_idx, const float* q_scale, const float* w, int64_t w_stride,
                                   const uint8_t* k_idx, const float* k_scale, const uint16_t* q, const void* kv,
                                   const float* kv_scale, int32_t kv_dtype, const int32_t* q_pos, int32_t n_q,
                                   int64_t n_k, int32_t h_idx, int32_t d_idx, int32_t top_k, float sm_scale,
                                   void* out, int32_t out_dtype, float* lse, int32_t* idx_out, void* ws,
                                   size_t ws_bytes, void* stream);

/*
 * sma_pcp_rank_share — one PCP rank's share of a prompt of L_total tokens
 * cut into 2*pcp_size equal chunks of C = L_total/(2*pcp_size) tokens
 * (same article, "PCP : répartir les tokens, pas les têtes": one early and
 * one late chunk per rank; the pair is (rank, 2*pcp_size-1-rank)).
 *
 *  The share's 2C query rows are chunk `rank` (positions rank*C ..) followed
 *  by chunk 2*pcp_size-1-rank; q_idx_share, w_share, q_share, out_share,
 *  lse_share and idx_share are indexed by these 2C rows.  k_idx and kv hold
 *  the whole gathered context (L_total rows).  The positions are built on
 *  the device in the workspace; the rest is sma_prefill.
 *  Requires 0 <= rank < pcp_size and L_total % (2*pcp_size) == 0.
 */
sma_status sma_pcp_rank_share(int32_t rank, int32_t pcp_size, int64_t L_total,
                              const uint16_t* q_idx_share, const float* w_share, int64_t w_stride,
                              const void* k_idx, const float* k_scale, int32_t k_dtype,
                              const uint16_t* q_share, const void* kv, const float* kv_scale,
                              int32_t kv_dtype, int32_t h_idx, int32_t d_idx, int32_t top_k,
                              float sm_scale, void* out_share, int32_t out_dtype, float* lse_share,
                              int32_t* idx_share, void* ws, size_t ws_bytes, void* stream);

/*
 * sma_absorb_q / sma_project_out — the absorbed form's per-head batched
 * products around sparse MLA (DeepSeek multi-node page, "Couche MLA":
 * kv_b_proj split into k_b_proj and v_b_proj, computed as batched products;
 * "Travaux futurs": decode absorbs the matrices).  With the key half
 * W_UK[h] and the value half W_UV[h] of kv_b_proj, each [128, 512] bf16
 * (row d of W_UK[h] maps the 512-dim latent to no-rope key dim d):
 *
 *   sma_absorb_q:    q_out[(i*heads + h)*ld_out + c] = sum_d q_nope[i,h,d] * W_UK[h,d,c]
 *                    for c < 512 (the rest of each ld_out row is untouched,
 *                    so ld_out = 576 writes the latent part of a sparse-MLA
 *                    query [n, heads, 576] in place, beside its rope dims)
 *   sma_project_out: out[i,h,d] = sum_c o_lat[i,h,c] * W_UV[h,d,c]
 *
 *  q_nope [n, heads, 128], w_uk / w_uv [heads, 128, 512], o_lat [n, heads,
 *  512], out [n, heads, 128]: bf16, contiguous, 16-byte aligned.  fp32
 *  accumulation on bf16 MFMA, one rounding to bf16 at the end.
 *  Requires 1 <= heads <= 1024, ld_out >= 512 and a multiple of 8.
 */
sma_status sma_absorb_q(const uint16_t* q_nope, const uint16_t* w_uk, int32_t n, int32_t heads, uint16_t* q_out,
                        int64_t ld_out, void* stream);
sma_status sma_project_out(const uint16_t* o_lat, const uint16_t* w_uv, int32_t n, int32_t heads, uint16_t* out,
                           void* stream);

/*
 * sma_dense_mha_prefill — dense causal multi-head attention over the latent
 * expanded per head: the prefill path for prompts that fit inside top-k
 * (GLM-5.3 part 2, "Essayez-le": without the forced MQA mode, prefill
 * batches whose prompts fit in the 2,048-token top-k take dense MHA;
 * DeepSeek multi-node page, "Travaux futurs": in prefill, project the latent
 * into K/V space first, then run MHA; "Couche MLA": kv_b_proj's key half
 * W_UK and value half W_UV).  For query i at p_i = clamp(q_pos[i], -1,
 * n_k-1) and head h, over s = 0..p_i:
 *
 *   k[s,h,:] = [W_UK[h] kv[s,0:512], kv[s,512:576]]   v[s,h,:] = W_UV[h] kv[s,0:512]
 *   out[i,h,:] = sum_s softmax_s(sm_scale * q[i,h,:] . k[s,h,:]) v[s,h,:]
 *   lse[i,h]   = log sum_s exp(sm_scale * q[i,h,:] . k[s,h,:])   (natural log)
 *
 *  q      [n_q, 64, 192] bf16: each head's 128 no-rope dims, then its 64
 *         rope dims
 *  kv     [n_k, 576] bf16 latent rows (the sparse path's KV)
 *  w_uk, w_uv [64, 128, 512] bf16 (row d of W_UK[h] maps the latent to
 *         no-rope key dim d, row d of W_UV[h] to value dim d; the layout of
 *         sma_absorb_q / sma_project_out)
 *  out    [n_q, 64, 128] bf16 or fp32 (out_dtype); lse [n_q, 64] fp32 or NULL.
 *         A query with an empty prefix (p_i = -1) gets 0 and -inf.
 *  ws     at least sma_workspace_bytes(SMA_OP_DENSE_MHA, n_q, n_k, ...) =
 *         n_k * 32,768 bytes, 256-byte aligned: the expanded keys and
 *         values, bf16 (one rounding each); fp32 accumulation and softmax.
 *  With every causal token selected (p_i < top_k, the prompts the pages
 *  route here) the result equals sma_project_out applied to
 *  sma_sparse_mla_prefill over the absorbed query [W_UK^T q_nope, q_rope],
 *  up to rounding; sm_scale must be finite and > 0.  Tensors 16-byte
 *  aligned.  n_q = 0 is a no-op.
 */
sma_status sma_dense_mha_prefill(const uint16_t* q, const uint16_t* kv, const uint16_t* w_uk, const uint16_t* w_uv,
                                 const int32_t* q_pos, int32_t n_q, int64_t n_k, float sm_scale, void* out,
                                 int32_t out_dtype, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * sma_dcp_shard_partial — one DCP rank's share of sparse MLA (same article,
 * "DCP : sharder aussi le cache KV": tokens are dealt round-robin over the
 * dcp_size ranks, so rank r stores tokens r, r + P, r + 2P, ...; in decode
 * each rank attends over its own shard and the partial results are merged
 * by their log-sum-exp, sma_lse_merge).
 *
 *  kv_local  [n_k_local, 576] the rank's shard: local row j is token
 *            j*dcp_size + rank (bf16, or e4m3fn codes with kv_scale_local)
 *  idx       [n_q, top_k] int32 global token positions of each query's
 *            selection (as sma_topk_select writes them); the rank keeps the
 *            entries it stores, other entries, negative ones and rows past
 *            the shard are skipped
 *  out_partial [n_q, 64, 512] fp32 and lse_partial [n_q, 64] fp32: the
 *            attention over the kept rows alone, normalised over them, as in
 *            sma_sparse_mla_prefill; a query the rank stores none of gets
 *            0 and -inf
 *  ws        at least sma_workspace_bytes(SMA_OP_DCP_PARTIAL, n_q, n_k_local,
 *            top_k, 0, 0) bytes, 256-byte aligned (the rank's local index
 *            list, and a small batch's row slices)
 *  Requires 0 <= rank < dcp_size.
 */
sma_status sma_dcp_shard_partial(int32_t rank, int32_t dcp_size, const uint16_t* q, const void* kv_local,
                                 const float* kv_scale_local, int32_t kv_dtype, int64_t n_k_local,
                                 const int32_t* idx, int32_t n_q, int32_t top_k, float sm_scale,
                                 float* out_partial, float* lse_partial, void* ws, size_t ws_bytes,
                                 void* stream);

/*
 * sma_dcp_shard_partial_noalloc — sma_dcp_shard_partial for callers that
 * cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): no workspace argument,
 * and no allocation inside.
 *
 *  Scratch: a static device array of SMA_STATIC_SCRATCH_BYTES (64 MiB) per
 *  device, part of the library's code object, so each device that runs the
 *  library holds it until the process ends.  It holds the rank's local
 *  index list (n_q*top_k*4 bytes, 256-byte aligned) and, in what remains,
 *  the partials of a small batch's row slices (as many slices as fit, up to
 *  the count sma_dcp_shard_partial uses with a full workspace).  With the
 *  same slice count the two entries give identical results; with fewer
 *  slices they differ by the bf16 rounding of the softmax weights, which
 *  each slice takes against its own running maximum (about 2^-8 relative).
 *  Every buffer is written before it is read, so nothing from an earlier
 *  call leaks into a result.
 *  Limit: a call whose index list exceeds the scratch (n_q*top_k >
 *  SMA_STATIC_SCRATCH_BYTES/4 = 16,777,216 entries) returns
 *  SMA_ERR_WORKSPACE before any launch.
 *  Concurrency: every call on one device shares that device's array.  Calls
 *  ordered on one stream are safe; calls that overlap in time on one device
 *  (different streams, or several host threads) race on it and give wrong
 *  results.
 *  Arguments, results and the other errors are those of
 *  sma_dcp_shard_partial.
 */
#define SMA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
sma_status sma_dcp_shard_partial_noalloc(int32_t rank, int32_t dcp_size, const uint16_t* q, const void* kv_local,
                                         const float* kv_scale_local, int32_t kv_dtype, int64_t n_k_local,
                                         const int32_t* idx, int32_t n_q, int32_t top_k, float sm_scale,
                                         float* out_partial, float* lse_partial, void* stream);

/*
 * sma_lse_merge — merge n_part partial attention results by their
 * log-sum-exp (same article and section):
 *   L[i,h]   = log(sum_r exp(lses[r,i,h]))
 *   out[i,h] = sum_r exp(lses[r,i,h] - L[i,h]) * parts[r,i,h,:]
 *  parts [n_part, n_q, 64, 512] fp32, lses [n_part, n_q, 64] fp32 (natural
 *  log, -inf for an empty partial); out [n_q, 64, 512] bf16 or fp32 (out_dtype);
 *  lse_out [n_q, 64] fp32 or NULL.  A (query, head) whose partials are all
 *  empty gets 0 and -inf.  Requires 1 <= n_part <= 64 and n_q <= 2^28.
 */
sma_status sma_lse_merge(const float* parts, const float* lses, int32_t n_part, int32_t n_q, void* out,
                         int32_t out_dtype, float* lse_out, void* stream);

/* Minimum workspace in bytes for `op` (an sma_op) at these sizes
 * (SMA_OP_DENSE_MHA: n_k * 64 * 256 * 2, whatever n_q and top_k).  For
 * SMA_OP_PREFILL / SMA_OP_PCP_SHARE, n_q is the number of query rows and the
 * figure assumes idx_out == NULL (the index list lives in the workspace).
 * For SMA_OP_SPARSE_MLA the workspace is optional: the figure is what lets a
 * small batch split its queries' rows (0 when no split is used). */
size_t sma_workspace_bytes(int32_t op, int32_t n_q, int64_t n_k, int32_t top_k,
                           int32_t h_idx, int32_t d_idx);

/* Message of the calling thread's last failed call ("" if none).  The
 * pointer stays valid until the thread's next call into the library. */
const char* sma_last_error(void);

/* ABI version: (major << 16) | minor. */
int32_t sma_version(void);

/* Build flags of the loaded library: SMA_BUILD_DEBUG_CHECKS in the debug
 * build (the device-resident range checks and workspace fill described at
 * the top of this file), 0 in the release build. */
#define SMA_BUILD_DEBUG_CHECKS 1
int32_t sma_build_flags(void);

#ifdef __cplusplus
}
#endif
#endif /* SMA_H */
