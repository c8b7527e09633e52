"""Algorithmic FLOP and byte counts for the sparse-MLA prefill path.

These are the method's own costs (what one launch must compute and move at
minimum), used for roofline fractions.  The per-row sparse-MLA accounting
follows footnote 1 of the GLM-5.3 part 2 article (PCP, DCP and Hybrid
HiSparse on 16 H200): QK over 576 dims plus PV over 512 dims per head and
selected row, bf16 q and o per head, a 4-byte index per selected row.
Footnote 3 of the same article gives the per-token FP8 KV budget; the
DeepSeek multi-node deployment page gives 70,272 bytes of bf16 latent per
token for 61 layers.
"""
from __future__ import annotations

import numpy as np

N_HEADS = 64
D_QK = 576
D_V = 512

# MI355X published peaks (dense, no sparsity)
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0


def mla_flops_per_head_row() -> int:
    """One head against one selected row: 2*576 (QK) + 2*512 (PV)."""
    return 2 * D_QK + 2 * D_V


def mla_qo_bytes_per_head(elem_bytes: int = 2) -> int:
    return (D_QK + D_V) * elem_bytes


def mla_query_intensity(heads: int, top_k: int = 2048, row_bytes: int = 656, index_bytes: int = 4):
    """(FLOPs, bytes, FLOPs/byte) of one query whose selected rows are read
    once and shared by ``heads`` heads."""
    flops = heads * mla_flops_per_head_row() * top_k
    byts = top_k * (row_bytes + index_bytes) + heads * mla_qo_bytes_per_head()
    return flops, byts, flops / byts


def glm_kv_bytes_per_token() -> int:
    """78 MLA layers x 656 B + 21 indexer layers x (128 FP8 + 4 B scale) + 788 B MTP."""
    return 78 * 656 + 21 * (128 + 4) + 788


def deepseek_latent_bytes_per_token(layers: int = 61) -> int:
    return layers * D_QK * 2


def ridge(tflops: float, tbs: float) -> float:
    return tflops / tbs


# ------------------------------------------------------------- workloads --

def causal_pairs(q_pos) -> int:
    """(query, key) pairs the indexer scores: sum of p_i + 1."""
    return int(np.sum(np.asarray(q_pos, dtype=np.int64) + 1))


def selected_rows(q_pos, top_k: int) -> int:
    return int(np.sum(np.minimum(np.asarray(q_pos, dtype=np.int64) + 1, top_k)))


def indexer_flops_per_pair(h_idx: int, d_idx: int) -> int:
    return 2 * h_idx * d_idx


def indexer_bytes(q_pos, h_idx: int, d_idx: int, key_bytes: int, score_bytes: int = 4) -> int:
    """Minimum HBM bytes of one index_scores launch: q_I (bf16) and w (fp32)
    read once per query, each key row read once, one fp32 score written per
    causal pair."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    n_q = q_pos.size
    n_k = int(q_pos.max()) + 1 if n_q else 0
    return n_q * h_idx * (2 * d_idx + 4) + n_k * key_bytes + causal_pairs(q_pos) * score_bytes


def indexer_bytes_per_request(q_pos, h_idx: int, d_idx: int, key_bytes: int, score_bytes: int = 4,
                              q_bytes_per_elem: int = 2) -> int:
    """HBM bytes of one index_scores launch when every query streams its own
    causal prefix of keys (the decode batch, where each request would own
    its KV): q_I and w once per query, key_bytes per causal pair read, one
    fp32 score written per causal pair.  FP8 queries (q_bytes_per_elem = 1)
    add a 4-byte scale per head row."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    q_row = q_bytes_per_elem * d_idx + (4 if q_bytes_per_elem == 1 else 0)
    return q_pos.size * h_idx * (q_row + 4) + causal_pairs(q_pos) * (key_bytes + score_bytes)


def topk_bytes(q_pos, top_k: int) -> int:
    """Minimum HBM bytes of one topk_select launch: every causal score read
    once, top_k int32 indices written per query."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    return causal_pairs(q_pos) * 4 + q_pos.size * top_k * 4


def mla_flops(q_pos, top_k: int, heads: int = N_HEADS) -> int:
    return selected_rows(q_pos, top_k) * heads * mla_flops_per_head_row()


def mla_bytes(q_pos, top_k: int, row_bytes: int, out_bytes: int, heads: int = N_HEADS) -> int:
    """Bytes one sparse_mla_prefill launch moves if every selected row is
    fetched once per query: rows + 4-byte indices + q (bf16) + output."""
    q_pos = np.asarray(q_pos, dtype=np.int64)
    n_q = q_pos.size
    return (selected_rows(q_pos, top_k) * row_bytes + n_q * top_k * 4
            + n_q * heads * (D_QK * 2 + D_V * out_bytes))


def flop_crossover_tokens(h_idx: int, d_idx: int, top_k: int, heads: int = N_HEADS) -> int:
    """Smallest prompt length L whose indexer FLOPs (every causal pair of
    positions 0 .. L-1) reach its sparse-MLA FLOPs (min(p + 1, top_k)
    selected rows per position).  Past top_k the indexer grows as L^2 and
    the attention as L, which is why the GLM-5.3 part 2 article ("Pourquoi
    pas TP ou DP ?") has the indexer overtake sparse MLA at some per-GPU
    prompt length."""
    def diff(L: int) -> int:
        pos = np.arange(L, dtype=np.int64)
        return causal_pairs(pos) * indexer_flops_per_pair(h_idx, d_idx) - mla_flops(pos, top_k, heads)

    lo, hi = 1, 1
    while diff(hi) < 0:
        lo, hi = hi, hi * 2
    while lo < hi:
        mid = (lo + hi) // 2
        if diff(mid) < 0:
            lo = mid + 1
        else:
            hi = mid
    return lo
