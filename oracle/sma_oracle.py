"""CPU oracle for the sparse-MLA prefill path: indexer -> top-k -> sparse MLA.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package entry's smoke check
and the bench's CPU-baseline leg may import this module.  The GPU library
never calls it and shares no code with it.

It is the method written out plainly, one query at a time, in float64
(the pages fix no precision; float64 is at least as accurate as the fp32
accumulation the GPU kernels use).  Library primitives (a matrix product,
``np.partition``, ``np.exp``) serve as steps; there is no blocking, fusion
or reordering beyond what each definition states.

Sources, by page and section:

* GLM-5.3 part 2 (PCP, DCP and Hybrid HiSparse on 16 H200), section
  "Pourquoi pas TP ou DP ?": the indexer scores every earlier token of the
  prompt and keeps the 2,048 that sparse MLA then reads.
* same page, section "PCP : répartir les tokens, pas les têtes": sparse MLA
  runs with every latent KV row serving all 64 heads; the prompt is cut into
  16 chunks and each of 8 GPUs takes one early and one late chunk.
* same page, section "Essayez-le": with the MQA mode forced, prompts that fit
  inside top-k still run sparse MLA (so sparse equals dense causal there).
* same page, footnote 1: QK runs over 576 dims, PV over 512; indices are
  4 bytes; q and o are bf16.
* same page, footnote 3: an FP8 key is 128 values plus a 4-byte scale.
* same page, footnote 1: FlashMLA's fp8_ds_mla KV row of 656 bytes (its
  layout, not given on the page, is taken from FlashMLA's public
  description: 512 e4m3 codes, 4 fp32 scales of 128 dims each, 64 bf16 rope
  values).
* DeepSeek multi-node deployment page, section "Quantification": activations
  are quantised on the fly with one scale per 128-element vector.
* GLM-5.3 part 2, section "DCP : sharder aussi le cache KV": tokens are dealt
  round-robin over the ranks, each rank attends over its own shard and the
  partial results are merged by their log-sum-exp.
* DeepSeek multi-node deployment page (Perplexity), sections
  "Parallélisme de tenseurs" and "Travaux futurs": the latent is shared by
  all heads; kv_b_proj maps it to each head; decode absorbs the projection.

Readings where the pages are silent (each also listed in the design notes):

* indexer score I[i,s] = sum_h w[i,h] * ReLU(q_I[i,h,:] . k_I[s,:]) for
  0 <= s <= p_i (the query's own token included), no bias, no scaling;
* top-k keeps the min(K, p_i+1) largest scores; ties at the threshold go to
  the lowest positions; the list is ascending by position, padded with -1;
  -0.0 and +0.0 are the same value; a NaN ranks below every number;
* attention scale tau = 1/sqrt(192); value = the first 512 latent dims;
  LSE is the natural-log log-sum-exp of the scaled logits;
* FP8 is OCP e4m3fn (bias 7, max 448, no infinities) times a per-token fp32
  scale; the oracle dequantises first, then runs the same steps;
* FP8 queries of the indexer carry one scale per (query, head) row, set to
  amax/448 with round-to-nearest-even codes (quantize_fp8_rows).

Pins: tests/test_oracle_*.py check each function against what the pages and
the mathematics fix (integer brute force, library routines for the dense and
non-absorbed special cases, invariants, the FP8 library cast, the pages'
printed byte and FLOP figures).

Parity unpinned: fp8_ds_mla_rows_to_f64 beyond the row's 656 bytes.  The
pages give only the size; the order of codes, scales and rope inside the
row is a reading of FlashMLA's description, and the test that checks the
decoder builds its rows from that same reading.
"""
from __future__ import annotations

import numpy as np

D_QK = 576
D_V = 512


# ---------------------------------------------------------------- storage --

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 is the upper half of an fp32: widen the 16 bits and reinterpret."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def e4m3fn_value(code: int) -> float:
    """Value of one OCP FP8 E4M3FN code: 1 sign, 4 exponent (bias 7),
    3 mantissa bits; exponent 0 is subnormal; S.1111.111 is NaN; no inf."""
    sign = -1.0 if (code >> 7) & 1 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3fn_table() -> np.ndarray:
    return np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


_E4M3 = e4m3fn_table()


def fp8_rows_to_f64(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Dequantise per-token FP8 rows: x[s, :] = e4m3(code[s, :]) * scale[s]
    (GLM-5.3 part 2, footnote 3: 128 FP8 values plus a 4-byte scale)."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)] * np.asarray(scale, dtype=np.float64)[:, None]


DS_ROW_BYTES = 656   # 512 e4m3 codes + 4 fp32 scales + 64 bf16 rope values


def fp8_ds_mla_rows_to_f64(rows: np.ndarray) -> np.ndarray:
    """Decode FlashMLA's 656-byte fp8_ds_mla latent rows (GLM-5.3 part 2,
    footnote 1, names the format and its 656 bytes; the layout is the one
    FlashMLA's public description gives): bytes 0..511 are the e4m3fn codes
    of latent dims 0..511, bytes 512..527 four little-endian fp32 scales,
    scale b for dims 128b .. 128b+127, and bytes 528..655 the 64 rope dims
    512..575 as bf16, unscaled.  rows uint8 [n, 656] -> float64 [n, 576].
    Parity unpinned beyond the 656 bytes (the pages do not give the layout)."""
    rows = np.ascontiguousarray(rows, dtype=np.uint8)
    if rows.ndim != 2 or rows.shape[1] != DS_ROW_BYTES:
        raise ValueError("fp8_ds_mla rows are uint8 [n, 656]")
    n = rows.shape[0]
    scales = rows[:, 512:528].copy().view("<f4").astype(np.float64)          # [n, 4]
    nope = _E4M3[rows[:, :512]] * np.repeat(scales, 128, axis=1)              # [n, 512]
    rope = bf16_bits_to_f64(rows[:, 528:656].copy().view("<u2"))              # [n, 64]
    return np.concatenate([nope, rope], axis=1).reshape(n, D_QK)


def keys_f64(k, fp8: bool) -> np.ndarray:
    return fp8_rows_to_f64(*k) if fp8 else bf16_bits_to_f64(k)


FP8_MAX = 448.0   # largest finite e4m3fn magnitude


def e4m3fn_encode(v) -> np.ndarray:
    """Nearest OCP E4M3FN code to each finite value with |v| <= 448, ties to
    the even code, the sign of zero kept.

    The format's grid, written out: in the binade [2^e, 2^(e+1)), e >= -6,
    the 8 codes are spaced 2^(e-3) apart; below 2^-6 the subnormals continue
    with spacing 2^-9.  So with e = max(floor(log2|v|), -6) and
    n = round_half_even(|v| / 2^(e-3)), the magnitude code is 8*(e+6) + n
    (n = 16, a value rounded up into the next binade, lands on that binade's
    first code).
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    if not np.all(a <= FP8_MAX):
        raise ValueError("e4m3fn_encode takes finite values with |v| <= 448")
    _, ex = np.frexp(a)                       # a = m * 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, -6)
    n = np.rint(a / np.ldexp(1.0, e - 3))     # np.rint: round half to even
    mag = np.where(a == 0, 0, 8 * (e + 6) + n).astype(np.int64)
    sign = np.signbit(v).astype(np.int64) << 7
    return (sign | mag).astype(np.uint8)


def quantize_fp8_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """Per-row FP8 quantisation of activations: one fp32 scale per row (the
    DeepSeek multi-node page, section "Quantification": activation scales are
    taken on the fly over vectors of 128 elements; an indexer head's q_I row
    is one such vector).  The decisions are taken in fp32, as the GPU takes
    them: scale = amax / 448, y = x / scale (both correctly rounded fp32
    divisions), y clamped to [-448, 448], code = nearest e4m3fn value.  A row
    of zeros gets scale 0 and zero codes.  x [n, d] (any float dtype, taken
    as fp32) -> codes uint8 [n, d], scale float32 [n]."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=1)
    scale = (amax / np.float32(FP8_MAX)).astype(np.float32)
    nz = scale > 0
    y = np.zeros_like(x)
    y[nz] = x[nz] / scale[nz][:, None]
    y = np.clip(y, -np.float32(FP8_MAX), np.float32(FP8_MAX))
    return e4m3fn_encode(y), scale


# ----------------------------------------------------------------- a1 -----

def index_scores(q_idx: np.ndarray, w: np.ndarray, k_idx: np.ndarray, q_pos: np.ndarray) -> list:
    """Indexer scores of each query over its causal prefix.

    q_idx [n_q, H_I, d_I] float64, w [n_q, H_I] float64, k_idx [n_k, d_I]
    float64, q_pos [n_q] int.  Returns a list: entry i is the float64 vector
    I[i, 0..p_i] with I[i,s] = sum_h w[i,h] * max(0, q_idx[i,h,:] . k_idx[s,:]).
    "Scores every earlier token" (GLM-5.3 part 2, "Pourquoi pas TP ou DP ?");
    the query's own position is included.
    """
    out = []
    for i in range(q_idx.shape[0]):
        p = int(q_pos[i])
        dots = q_idx[i] @ k_idx[: p + 1].T          # [H_I, p+1]
        out.append(w[i] @ np.maximum(dots, 0.0))    # [p+1]
    return out


def index_scores_fp8(q8: np.ndarray, q_scale: np.ndarray, w: np.ndarray, k8: np.ndarray,
                     k_scale: np.ndarray, q_pos: np.ndarray) -> list:
    """Indexer scores with FP8 queries and FP8 keys: q_I[i,h,:] =
    e4m3(q8[i,h,:]) * q_scale[i,h] (one scale per head row of 128 values, the
    DeepSeek page's activation blocks) and k_I[s,:] = e4m3(k8[s,:]) *
    k_scale[s] (GLM-5.3 part 2, footnote 3); then index_scores on the
    dequantised values.  q8 uint8 [n_q, H_I, d_I], q_scale [n_q, H_I]."""
    n_q, h, d = q8.shape
    q = fp8_rows_to_f64(np.asarray(q8).reshape(n_q * h, d), np.asarray(q_scale).reshape(-1))
    return index_scores(q.reshape(n_q, h, d), np.asarray(w, dtype=np.float64),
                        fp8_rows_to_f64(k8, k_scale), q_pos)


# ----------------------------------------------------------------- a2 -----

def topk_row(scores: np.ndarray, top_k: int) -> np.ndarray:
    """Top-k of one causal row (positions 0..len-1), ascending, -1 padded.

    Keeps m = min(top_k, len) positions: every position whose score is above
    the m-th largest value T, then the lowest positions whose score equals T
    until m are kept.  A NaN score ranks below every number (-inf included):
    NaN positions are kept only when fewer than m scores are numbers, the
    lowest NaN positions first.
    """
    s = np.asarray(scores, dtype=np.float64)
    n = s.size
    m = min(top_k, n)
    out = np.full(top_k, -1, dtype=np.int32)
    if m == 0:
        return out
    nan = np.isnan(s)
    num = np.flatnonzero(~nan)                      # positions holding numbers
    if num.size >= m:
        v = s[num]
        t = np.partition(v, v.size - m)[v.size - m]   # m-th largest number
        above = num[v > t]
        ties = num[v == t][: m - above.size]
        sel = np.concatenate([above, ties])
    else:
        sel = np.concatenate([num, np.flatnonzero(nan)[: m - num.size]])
    out[:m] = np.sort(sel)
    return out


def topk_select(score_rows: list, top_k: int) -> np.ndarray:
    return np.stack([topk_row(r, top_k) for r in score_rows]) if score_rows else \
        np.zeros((0, top_k), dtype=np.int32)


def topk_threshold(scores: np.ndarray, top_k: int) -> float:
    """The m-th largest score of a row (the value the selection is cut at)."""
    s = np.asarray(scores, dtype=np.float64)
    m = min(top_k, s.size)
    return float(np.partition(s, s.size - m)[s.size - m])


# ----------------------------------------------------------------- a4 -----

def sparse_mla(q: np.ndarray, kv: np.ndarray, idx: np.ndarray, sm_scale: float):
    """Absorbed (MQA-mode) sparse MLA over each query's selected latent rows.

    q [n_q, H, 576] float64, kv [n_k, 576] float64, idx [n_q, K] int
    (negative entries are padding).  For each query i and head h over the
    selected set S_i: z_s = tau * q[i,h,:] . kv[s,:576];
    o[i,h,:] = sum_s softmax(z)_s * kv[s,:512]; lse[i,h] = log sum_s exp(z_s).
    One latent row serves all heads (GLM-5.3 part 2, "PCP : répartir les
    tokens, pas les têtes"); QK over 576, PV over 512 (footnote 1).
    An empty set gives o = 0 and lse = -inf.
    """
    n_q, n_h, _ = q.shape
    out = np.zeros((n_q, n_h, D_V), dtype=np.float64)
    lse = np.full((n_q, n_h), -np.inf, dtype=np.float64)
    for i in range(n_q):
        sel = idx[i][idx[i] >= 0]
        if sel.size == 0:
            continue
        rows = kv[sel]                               # [m, 576]
        z = sm_scale * (q[i] @ rows.T)               # [H, m]
        mx = z.max(axis=1, keepdims=True)
        e = np.exp(z - mx)
        den = e.sum(axis=1, keepdims=True)
        out[i] = (e @ rows[:, :D_V]) / den
        lse[i] = mx[:, 0] + np.log(den[:, 0])
    return out, lse


# --------------------------------------------------------------- compose --

def prefill(q_idx, w, k_idx, q, kv, q_pos, top_k: int, sm_scale: float):
    """indexer -> top-k -> sparse MLA for the given query rows (float64 in)."""
    scores = index_scores(q_idx, w, k_idx, q_pos)
    idx = topk_select(scores, top_k)
    out, lse = sparse_mla(q, kv, idx, sm_scale)
    return scores, idx, out, lse


def absorb_q(q_nope: np.ndarray, w_uk: np.ndarray) -> np.ndarray:
    """Absorb the key half of kv_b_proj into the query (DeepSeek multi-node
    page, "Couche MLA": kv_b_proj split into k_b_proj and v_b_proj, computed
    as batched products; "Travaux futurs": decode absorbs the matrices).  A
    head's no-rope key is k[s,h,:] = W_UK[h] c_s, so q_nope[i,h,:] . k[s,h,:]
    = (W_UK[h]^T q_nope[i,h,:]) . c_s:  q_lat[i,h,:] = W_UK[h]^T q_nope[i,h,:].
    q_nope [n, H, d_nope], w_uk [H, d_nope, d_lat] -> [n, H, d_lat]."""
    return np.einsum("nhd,hdc->nhc", np.asarray(q_nope, np.float64), np.asarray(w_uk, np.float64))


def project_out(o_lat: np.ndarray, w_uv: np.ndarray) -> np.ndarray:
    """Apply the value half of kv_b_proj to the attention's latent output
    (same page and sections): v[s,h,:] = W_UV[h] c_s, so the head's output is
    o[i,h,:] = W_UV[h] o_lat[i,h,:].  o_lat [n, H, d_lat], w_uv [H, d_v,
    d_lat] -> [n, H, d_v]."""
    return np.einsum("nhc,hvc->nhv", np.asarray(o_lat, np.float64), np.asarray(w_uv, np.float64))


def dense_mha_prefill(q_mha: np.ndarray, kv: np.ndarray, w_uk: np.ndarray, w_uv: np.ndarray, q_pos,
                      sm_scale: float):
    """Dense causal multi-head attention over the latent expanded per head:
    the prefill path the pages describe for prompts that fit inside top-k
    (GLM-5.3 part 2, "Essayez-le": without the forced MQA mode, such prefill
    batches take the dense MHA path; DeepSeek multi-node page, "Travaux
    futurs": in prefill, project the latent into K/V space first, then run
    multi-head attention; "Couche MLA": kv_b_proj split into its key and
    value halves).

    q_mha [n_q, H, 192]: each head's 128 no-rope dims then its 64 rope dims;
    kv [n_k, 576]: latent c_s (dims 0..511) and the shared rope key (dims
    512..575); w_uk, w_uv [H, 128, 512] (row d of W_UK[h] maps the latent to
    no-rope key dim d, row d of W_UV[h] to value dim d).  For query i at
    position p_i and head h, over s = 0..p_i:
        k[s,h,:] = [W_UK[h] c_s, rope_s]      v[s,h,:] = W_UV[h] c_s
        z_s = tau * q_mha[i,h,:] . k[s,h,:]
        o[i,h,:] = sum_s softmax(z)_s v[s,h,:],  lse[i,h] = log sum_s exp(z_s)
    Returns (o [n_q, H, 128], lse [n_q, H]); an empty prefix (p_i < 0)
    gives o = 0 and lse = -inf.
    """
    q_mha = np.asarray(q_mha, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    w_uk = np.asarray(w_uk, dtype=np.float64)
    w_uv = np.asarray(w_uv, dtype=np.float64)
    n_q, n_h, _ = q_mha.shape
    d_nope = w_uk.shape[1]
    c, rope = kv[:, :D_V], kv[:, D_V:]
    # per head h: k_nope[h, s, :] = W_UK[h] c_s and v[h, s, :] = W_UV[h] c_s
    k_nope = np.matmul(w_uk, c.T).transpose(0, 2, 1)   # [H, n_k, 128]: the key half of kv_b_proj
    v = np.matmul(w_uv, c.T).transpose(0, 2, 1)        # [H, n_k, 128]: the value half
    out = np.zeros((n_q, n_h, w_uv.shape[1]), dtype=np.float64)
    lse = np.full((n_q, n_h), -np.inf, dtype=np.float64)
    for i in range(n_q):
        p = int(q_pos[i])
        if p < 0:
            continue
        qn, qr = q_mha[i, :, :d_nope], q_mha[i, :, d_nope:]
        z_nope = np.matmul(k_nope[:, : p + 1, :], qn[:, :, None])[:, :, 0]      # [H, p+1]
        z = sm_scale * (z_nope + qr @ rope[: p + 1].T)
        mx = z.max(axis=1, keepdims=True)
        e = np.exp(z - mx)
        den = e.sum(axis=1, keepdims=True)
        out[i] = np.matmul(e[:, None, :], v[:, : p + 1, :])[:, 0, :] / den     # [H, 128]
        lse[i] = mx[:, 0] + np.log(den[:, 0])
    return out, lse


def dcp_shard_rows(rank: int, dcp_size: int, kv: np.ndarray) -> np.ndarray:
    """The latent rows one DCP rank stores: tokens are dealt round-robin over
    the ranks, so rank r holds tokens r, r + P, r + 2P, ... (local row j is
    token j*P + r) (GLM-5.3 part 2, "DCP : sharder aussi le cache KV")."""
    if not (0 <= rank < dcp_size):
        raise ValueError("rank out of range")
    return kv[rank::dcp_size]


def dcp_shard_partial(rank: int, dcp_size: int, q: np.ndarray, kv: np.ndarray, idx: np.ndarray,
                      sm_scale: float):
    """One DCP rank's partial attention: over the selected tokens it stores
    (those s in S_i with s mod P = rank), the same softmax attention as
    sparse_mla, with its own normaliser; a query none of whose tokens the
    rank stores gets o = 0 and lse = -inf.  In decode each rank attends over
    its own shard and the partial results are merged by their log-sum-exp
    (same page and section).  kv is the whole context here; the rank reads
    the same rows from its shard (dcp_shard_rows)."""
    if not (0 <= rank < dcp_size):
        raise ValueError("rank out of range")
    idx = np.asarray(idx)
    own = np.where((idx >= 0) & (idx % dcp_size == rank), idx, -1)
    return sparse_mla(q, kv, own, sm_scale)


def lse_merge(parts: np.ndarray, lses: np.ndarray):
    """Merge partial attentions by log-sum-exp (same page and section): with
    L = log sum_r exp(lse_r), o = sum_r exp(lse_r - L) * o_r and the merged
    log-sum-exp is L.  parts [P, n_q, H, D], lses [P, n_q, H]; a (query,
    head) whose partials are all empty (lse = -inf) gets o = 0, L = -inf."""
    parts = np.asarray(parts, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    m = lses.max(axis=0)                                   # [n_q, H]
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    a = np.where(np.isfinite(lses), np.exp(lses - m_safe[None]), 0.0)   # [P, n_q, H]
    s = a.sum(axis=0)
    out = np.zeros(parts.shape[1:], dtype=np.float64)
    lse = np.full(m.shape, -np.inf, dtype=np.float64)
    w = np.where(finite[None], a / np.where(finite, s, 1.0)[None], 0.0)
    out[...] = np.einsum("pqh,pqhd->qhd", w, parts)
    lse[finite] = m[finite] + np.log(s[finite])
    return out, lse


def pcp_positions(rank: int, pcp_size: int, L_total: int) -> np.ndarray:
    """Query positions of one PCP rank: the prompt is cut into 2*pcp_size
    equal chunks and rank r takes chunk r and chunk 2*pcp_size-1-r, in that
    order (GLM-5.3 part 2, "PCP : répartir les tokens, pas les têtes"; the
    page's figure text naming the pair is lost, the pair (r, 15-r) for 8
    ranks is the plain reading of 'one early and one late chunk')."""
    nchunk = 2 * pcp_size
    if not (0 <= rank < pcp_size) or L_total % nchunk:
        raise ValueError("rank out of range or L_total not divisible by 2*pcp_size")
    c = L_total // nchunk
    return np.concatenate([np.arange(rank * c, (rank + 1) * c),
                           np.arange((nchunk - 1 - rank) * c, (nchunk - rank) * c)]).astype(np.int32)


def pcp_rank_share(rank: int, pcp_size: int, q_idx_full, w_full, k_idx, q_full, kv,
                   top_k: int, sm_scale: float):
    """One rank's share: rows of the full prompt at pcp_positions(rank),
    run through the same three steps against the whole causal context."""
    pos = pcp_positions(rank, pcp_size, k_idx.shape[0])
    return prefill(q_idx_full[pos], w_full[pos], k_idx, q_full[pos], kv, pos, top_k, sm_scale)
