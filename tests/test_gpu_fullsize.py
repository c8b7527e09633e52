"""GPU parity at the full sizes the bench times, in its launch configuration
(all query rows in one call): the 16,384- and 65,536-token prefills, the
64-query decode batch over a 1,048,576-token FP8 context and the
131,072-token PCP8 share at ranks 0 and 7, checked on sampled rows
against the oracle (threshold rule for the selections, attention on the
GPU's own lists within the bf16 / FP8 tolerance)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_index_amd as sma
from sparse_mla_attention_index_amd import synth
from _gpuhelp import check_topk_threshold_rule, host, out_f64

pytestmark = pytest.mark.gpu


def _upload(w, tensor, n, chunk, start=0):
    """Rows [start, start + n) of a workload tensor, generated in chunks
    straight into device memory (bf16 bits as int16; FP8 as codes + scales)."""
    first = synth.rows(w, tensor, start, start + min(n, chunk))
    if isinstance(first, tuple):
        codes = torch.empty((n,) + first[0].shape[1:], dtype=torch.uint8, device="cuda:0")
        scale = torch.empty((n,), dtype=torch.float32, device="cuda:0")
        out = (codes, scale)
    else:
        dt = torch.float32 if first.dtype == np.float32 else torch.int16
        out = torch.empty((n,) + first.shape[1:], dtype=dt, device="cuda:0")
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        x = first if a == 0 else synth.rows(w, tensor, start + a, start + b)
        if isinstance(x, tuple):
            out[0][a:b].copy_(torch.from_numpy(x[0]))
            out[1][a:b].copy_(torch.from_numpy(x[1]))
        else:
            out[a:b].copy_(torch.from_numpy(x.view(np.int16) if x.dtype == np.uint16 else x))
    return out


@pytest.mark.parametrize("cfg,rows", [
    (2, [0, 1, 2047, 2048, 2049, 9999, 16382, 16383]),
    (3, [0, 2046, 2047, 2048, 31337, 65534, 65535]),
])
def test_prefill_full_size_sampled_rows(cfg, rows):
    """The 16K and 64K prompts: rows at both ends, and on both sides of the
    point where the causal prefix outgrows top_k (from 2,048 keys on, the
    selection is a strict subset)."""
    w = synth.workload(cfg)
    n = w.n_keys
    k_idx = _upload(w, "k_idx", n, 65536)
    kv = _upload(w, "kv", n, 16384)
    q_idx = _upload(w, "q_idx", n, 1024)
    wt = _upload(w, "w", n, 65536)
    q = _upload(w, "q", n, 256)
    pos = torch.arange(n, dtype=torch.int32, device="cuda:0")
    idx = torch.empty((n, w.top_k), dtype=torch.int32, device="cuda:0")
    # the bench's configuration: one score block holding every row
    ws = torch.empty(n * n * 4 + 4096, dtype=torch.uint8, device="cuda:0")
    out, lse, _ = sma.prefill(q_idx, wt, k_idx, q, kv, pos, w.top_k, w.sm_scale, want_lse=True, idx_out=idx,
                              workspace=ws)
    del ws
    torch.cuda.synchronize()
    rows = np.array(rows)
    sel = torch.from_numpy(rows).to("cuda:0")
    f = oracle.bf16_bits_to_f64
    kk = f(host(k_idx).view(np.uint16))
    kvv = f(host(kv).view(np.uint16))
    qi = f(host(q_idx[sel]).view(np.uint16))
    sc = oracle.index_scores(qi, host(wt[sel]).astype(np.float64), kk, rows)
    gi = host(idx[sel])
    for j, s in enumerate(sc):
        check_topk_threshold_rule(gi[j], s, w.top_k)
    ref, ref_lse = oracle.sparse_mla(f(host(q[sel]).view(np.uint16)), kvv, gi, w.sm_scale)
    got = out_f64(out[sel])
    assert np.abs(got - ref).max() <= 1e-2 * np.abs(ref).max()
    assert np.abs(host(lse[sel]) - ref_lse).max() < 2e-3


def test_decode_1m_fp8_sampled_queries():
    w = synth.workload(5)
    n_k = w.n_keys
    k8, ks = _upload(w, "k_idx", n_k, 65536)
    kv8, kvs = _upload(w, "kv", n_k, 65536)
    pos_np = synth.query_positions(w)
    q_idx = torch.from_numpy(synth.query_rows(w, "q_idx", pos_np).view(np.int16)).to("cuda:0")
    wt = torch.from_numpy(synth.query_rows(w, "w", pos_np)).to("cuda:0")
    q = torch.from_numpy(synth.query_rows(w, "q", pos_np).view(np.int16)).to("cuda:0")
    pos = torch.from_numpy(pos_np).to("cuda:0")
    n_q = pos_np.size
    idx = torch.empty((n_q, w.top_k), dtype=torch.int32, device="cuda:0")
    out, lse, _ = sma.prefill(q_idx, wt, k8, q, kv8, pos, w.top_k, w.sm_scale, k_scale=ks, kv_scale=kvs,
                              want_lse=True, idx_out=idx)
    torch.cuda.synchronize()
    rows = np.array([0, 17, 40, n_q - 1])
    sel = torch.from_numpy(rows).to("cuda:0")
    f = oracle.bf16_bits_to_f64
    kk = oracle.fp8_rows_to_f64(host(k8), host(ks))
    sc = oracle.index_scores(f(host(q_idx[sel]).view(np.uint16)), host(wt[sel]).astype(np.float64), kk,
                             pos_np[rows])
    gi = host(idx[sel])
    for j, s in enumerate(sc):
        check_topk_threshold_rule(gi[j], s, w.top_k)
    used = np.unique(gi[gi >= 0])
    kv_used = oracle.fp8_rows_to_f64(host(kv8[torch.from_numpy(used).to("cuda:0")]),
                                     host(kvs[torch.from_numpy(used).to("cuda:0")]))
    remap = np.where(gi >= 0, np.searchsorted(used, np.maximum(gi, 0)), -1)
    ref, ref_lse = oracle.sparse_mla(f(host(q[sel]).view(np.uint16)), kv_used, remap, w.sm_scale)
    got = out_f64(out[sel])
    assert np.abs(got - ref).max() <= 3e-2 * np.abs(ref).max()
    assert np.abs(host(lse[sel]) - ref_lse).max() < 5e-3


def test_pcp_share_131k_ranks_0_and_7():
    """One PCP8 rank's share of a 131,072-token prompt (16 chunks of 8,192),
    ranks 0 and 7 in the bench's configuration (one score block holding all
    16,384 query rows), checked on rows at both chunks' first and last
    positions and spread between: the selections follow the threshold rule
    against the oracle's scores, attention on the GPU's own lists is within
    1e-2 of max|ref| and the LSE within 2e-3."""
    w = synth.workload(4)
    L, P = w.n_keys, w.pcp_size
    C = L // (2 * P)
    k_idx = _upload(w, "k_idx", L, 65536)
    kv = _upload(w, "kv", L, 16384)
    f = oracle.bf16_bits_to_f64
    kk = f(host(k_idx).view(np.uint16))
    kvv = f(host(kv).view(np.uint16))
    rows = np.unique(np.r_[0, 1, C - 1, C, C + 1, 2 * C - 2, 2 * C - 1,
                           np.linspace(0, 2 * C - 1, 7).round().astype(int)])
    sel = torch.from_numpy(rows).to("cuda:0")
    for r in (0, 7):
        pos_np = oracle.pcp_positions(r, P, L)
        halves = [(r * C, C), ((2 * P - 1 - r) * C, C)]
        q_idx = torch.cat([_upload(w, "q_idx", n, 1024, a) for a, n in halves])
        wt = torch.cat([_upload(w, "w", n, 65536, a) for a, n in halves])
        q = torch.cat([_upload(w, "q", n, 256, a) for a, n in halves])
        idx = torch.empty((2 * C, w.top_k), dtype=torch.int32, device="cuda:0")
        ws_n = 2 * C * 4 + 2 * C * L * 4 + sma.workspace_bytes(sma._lib.SMA_OP_TOPK, 2 * C, L, w.top_k) + 4096
        ws = torch.empty(ws_n, dtype=torch.uint8, device="cuda:0")
        out, lse, _ = sma.pcp_rank_share(r, P, q_idx, wt, k_idx, q, kv, w.top_k, w.sm_scale, want_lse=True,
                                         idx_share=idx, workspace=ws)
        torch.cuda.synchronize()
        del ws
        sub = pos_np[rows]
        sc = oracle.index_scores(f(host(q_idx[sel]).view(np.uint16)), host(wt[sel]).astype(np.float64), kk, sub)
        gi = host(idx[sel])
        for j, s_ in enumerate(sc):
            check_topk_threshold_rule(gi[j], s_, w.top_k)
        ref, ref_lse = oracle.sparse_mla(f(host(q[sel]).view(np.uint16)), kvv, gi, w.sm_scale)
        got = out_f64(out[sel])
        assert np.abs(got - ref).max() <= 1e-2 * np.abs(ref).max(), r
        assert np.abs(host(lse[sel]) - ref_lse).max() < 2e-3, r
        del q_idx, wt, q, out, lse, idx
        torch.cuda.empty_cache()
