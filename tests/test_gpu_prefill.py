"""GPU parity of the composed path (sma_prefill) and the PCP rank share."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_index_amd as sma
from sparse_mla_attention_index_amd import synth
from _gpuhelp import check_topk_threshold_rule, dev, host, out_f64

pytestmark = pytest.mark.gpu


def _load(w, n, positions=None):
    pos = np.arange(n, dtype=np.int32) if positions is None else positions
    d = dict(q_idx=synth.query_rows(w, "q_idx", pos), w=synth.query_rows(w, "w", pos),
             q=synth.query_rows(w, "q", pos), k_idx=synth.rows(w, "k_idx", 0, n),
             kv=synth.rows(w, "kv", 0, n), pos=pos)
    return d


def _gpu_prefill(w, d, want_idx=True, out_dtype=None):
    out_dtype = out_dtype or (torch.float32 if w.out_fp32 else torch.bfloat16)
    idx = torch.empty((d["pos"].size, w.top_k), dtype=torch.int32, device="cuda:0") if want_idx else None
    kk, kv = dev(d["k_idx"]), dev(d["kv"])
    ks = vs = None
    if isinstance(kk, tuple):
        kk, ks = kk
    if isinstance(kv, tuple):
        kv, vs = kv
    out, lse, _ = sma.prefill(dev(d["q_idx"]), dev(d["w"]), kk, dev(d["q"]), kv, dev(d["pos"]), w.top_k,
                              w.sm_scale, k_scale=ks, kv_scale=vs, out_dtype=out_dtype, want_lse=True,
                              idx_out=idx)
    torch.cuda.synchronize()
    return out, lse, idx


def test_tiny_workload_end_to_end():
    """Tiny workload: integer indexer -> the index lists are exact; the
    attention output (fp32) is within 1e-2 of max|ref|."""
    w = synth.workload(1)
    d = _load(w, w.n_keys)
    out, lse, idx = _gpu_prefill(w, d)
    f = oracle.bf16_bits_to_f64
    _, ref_idx, ref_out, ref_lse = oracle.prefill(f(d["q_idx"]), d["w"].astype(np.float64), f(d["k_idx"]),
                                                  f(d["q"]), f(d["kv"]), d["pos"], w.top_k, w.sm_scale)
    assert np.array_equal(host(idx), ref_idx)
    got = out_f64(out)
    assert np.abs(got - ref_out).max() <= 1e-2 * np.abs(ref_out).max()
    assert np.abs(got - ref_out).max() <= 2e-3 * np.abs(ref_out).max()
    assert np.abs(host(lse) - ref_lse).max() < 2e-3


def test_prefill_normal_inputs_threshold_rule():
    """16K-workload distributions at L=3000 (ragged): selections follow the
    1e-3 threshold rule; attention on the GPU's own lists is within 1e-2."""
    w = synth.workload(2)
    n = 3000
    d = _load(w, n)
    out, lse, idx = _gpu_prefill(w, d)
    f = oracle.bf16_bits_to_f64
    qi, kk = f(d["q_idx"]), f(d["k_idx"])
    gi = host(idx)
    rows = list(range(0, n, 29)) + [n - 1]
    sc = oracle.index_scores(qi[rows], d["w"][rows].astype(np.float64), kk, d["pos"][rows])
    ndiff = 0
    for r, s in zip(rows, sc):
        ndiff += check_topk_threshold_rule(gi[r], s, w.top_k)
    ref_out, _ = oracle.sparse_mla(f(d["q"][rows]), f(d["kv"]), gi[rows], w.sm_scale)
    got = out_f64(out)[rows]
    assert np.abs(got - ref_out).max() <= 1e-2 * np.abs(ref_out).max()


def test_prefill_deterministic_and_workspace_independent():
    w = synth.workload(2)
    d = _load(w, 1500)
    a = _gpu_prefill(w, d)
    # minimum workspace: score blocks of 64 rows instead of all rows at once
    kk, kv = dev(d["k_idx"]), dev(d["kv"])
    ws_min = sma.workspace_bytes(3, 1500, 1500, w.top_k)
    ws = torch.empty(ws_min, dtype=torch.uint8, device="cuda:0")
    idx = torch.empty((1500, w.top_k), dtype=torch.int32, device="cuda:0")
    out, lse, _ = sma.prefill(dev(d["q_idx"]), dev(d["w"]), kk, dev(d["q"]), kv, dev(d["pos"]), w.top_k,
                              w.sm_scale, want_lse=True, idx_out=idx, workspace=ws)
    assert torch.equal(a[2], idx) and torch.equal(a[0], out) and torch.equal(a[1], lse)


@pytest.mark.parametrize("kind", [1, 2])
def test_pcp_union_equals_unsharded(kind):
    """8 rank shares of a prompt cut into 16 chunks reproduce the unsharded
    prefill bit for bit."""
    base = synth.workload(kind)
    L = 2048 if kind == 1 else 4096
    w = base
    d = _load(w, L)
    out_full, lse_full, idx_full = _gpu_prefill(w, d)
    kk, kv = dev(d["k_idx"]), dev(d["kv"])
    seen = np.zeros(L, bool)
    for r in range(8):
        pos = oracle.pcp_positions(r, 8, L)
        idx = torch.empty((pos.size, w.top_k), dtype=torch.int32, device="cuda:0")
        out, lse, _ = sma.pcp_rank_share(r, 8, dev(d["q_idx"][pos]), dev(d["w"][pos]), kk, dev(d["q"][pos]), kv,
                                         w.top_k, w.sm_scale, out_dtype=out_full.dtype, want_lse=True,
                                         idx_share=idx)
        sel = torch.from_numpy(pos.astype(np.int64)).to("cuda:0")
        assert torch.equal(idx, idx_full[sel]), r
        assert torch.equal(out, out_full[sel]), r
        assert torch.equal(lse, lse_full[sel]), r
        seen[pos] = True
    assert seen.all()


def _gpu_share(w, d, r, P):
    pos = oracle.pcp_positions(r, P, d["pos"].size)
    idx = torch.empty((pos.size, w.top_k), dtype=torch.int32, device="cuda:0")
    out, lse, _ = sma.pcp_rank_share(r, P, dev(d["q_idx"][pos]), dev(d["w"][pos]), dev(d["k_idx"]),
                                     dev(d["q"][pos]), dev(d["kv"]), w.top_k, w.sm_scale,
                                     out_dtype=torch.float32 if w.out_fp32 else torch.bfloat16, want_lse=True,
                                     idx_share=idx)
    torch.cuda.synchronize()
    return pos, out, lse, idx


def test_pcp_shares_match_oracle_integer():
    """Every share of a 2,048-token prompt of the tiny workload's integer
    indexer (8 ranks, 16 chunks of 128) against oracle.pcp_rank_share: the
    index lists are identical (exact fp32 scores), the fp32 output and the
    LSE within 2e-3."""
    w = synth.workload(1)
    L, P = 2048, 8
    d = _load(w, L)
    f = oracle.bf16_bits_to_f64
    full = dict(qi=f(d["q_idx"]), w=d["w"].astype(np.float64), k=f(d["k_idx"]), q=f(d["q"]), kv=f(d["kv"]))
    for r in range(P):
        pos, out, lse, idx = _gpu_share(w, d, r, P)
        _, ref_idx, ref_out, ref_lse = oracle.pcp_rank_share(r, P, full["qi"], full["w"], full["k"], full["q"],
                                                             full["kv"], w.top_k, w.sm_scale)
        assert np.array_equal(host(idx), ref_idx), r
        got = out_f64(out)
        assert np.abs(got - ref_out).max() <= 2e-3 * np.abs(ref_out).max(), r
        assert np.abs(host(lse) - ref_lse).max() < 2e-3, r


def test_pcp_shares_match_oracle_normal():
    """Shares of a 4,096-token prompt with the 16K workload's N(0,1)
    distributions, ranks 0, 3 and 7: on rows at both chunks' edges and spread
    between, the selections follow the 1e-3 threshold rule against
    oracle.pcp_rank_share's scores; attention on the GPU's own lists is
    within 1e-2 of max|ref| and the LSE within 2e-3."""
    w = synth.workload(2)
    L, P = 4096, 8
    C = L // (2 * P)
    d = _load(w, L)
    f = oracle.bf16_bits_to_f64
    kk, kvv = f(d["k_idx"]), f(d["kv"])
    rows = np.unique(np.r_[0, 1, C - 1, C, C + 1, 2 * C - 1, np.linspace(0, 2 * C - 1, 10).round().astype(int)])
    for r in (0, 3, 7):
        pos, out, lse, idx = _gpu_share(w, d, r, P)
        assert np.array_equal(pos, np.r_[np.arange(r * C, (r + 1) * C), np.arange((2 * P - 1 - r) * C,
                                                                                   (2 * P - r) * C)])
        sub = pos[rows]
        sc = oracle.index_scores(f(d["q_idx"][sub]), d["w"][sub].astype(np.float64), kk, sub)
        gi = host(idx)[rows]
        for j, s in enumerate(sc):
            check_topk_threshold_rule(gi[j], s, w.top_k)
        ref, ref_lse = oracle.sparse_mla(f(d["q"][sub]), kvv, gi, w.sm_scale)
        got = out_f64(out)[rows]
        assert np.abs(got - ref).max() <= 1e-2 * np.abs(ref).max(), r
        assert np.abs(host(lse)[rows] - ref_lse).max() < 2e-3, r


@pytest.mark.parametrize("n_k", [100, 70000])
@pytest.mark.parametrize("n_q", [3, 8])
def test_prefill_small_batch_minimum_workspace(n_q, n_k):
    """A batch of fewer than 16 query rows on exactly the minimum workspace
    (sma_workspace_bytes(SMA_OP_PREFILL, ...), what the binding allocates by
    default), with rows shorter and longer than 65,536 scores: integer
    indexer inputs, so the lists equal the oracle's; fp32 output within
    2e-3 of max|ref|."""
    w = synth.workload(1)
    pos = np.array([n_k - 1, n_k // 2, 0, n_k - 2, 7, n_k // 3, 127, 128][:n_q], dtype=np.int32)
    d = dict(q_idx=synth.query_rows(w, "q_idx", pos), w=synth.query_rows(w, "w", pos),
             q=synth.query_rows(w, "q", pos), k_idx=synth.rows(w, "k_idx", 0, n_k), kv=synth.rows(w, "kv", 0, n_k),
             pos=pos)
    ws_min = sma.workspace_bytes(sma._lib.SMA_OP_PREFILL, n_q, n_k, w.top_k, w.h_idx, w.d_idx)
    ws = torch.empty(ws_min, dtype=torch.uint8, device="cuda:0")
    idx = torch.empty((n_q, w.top_k), dtype=torch.int32, device="cuda:0")
    out, lse, _ = sma.prefill(dev(d["q_idx"]), dev(d["w"]), dev(d["k_idx"]), dev(d["q"]), dev(d["kv"]),
                              dev(d["pos"]), w.top_k, w.sm_scale, out_dtype=torch.float32, want_lse=True,
                              idx_out=idx, workspace=ws)
    # the same call with the index list kept inside that workspace (idx_out
    # NULL: the figure sma_workspace_bytes assumes)
    out2, lse2, _ = sma.prefill(dev(d["q_idx"]), dev(d["w"]), dev(d["k_idx"]), dev(d["q"]), dev(d["kv"]),
                                dev(d["pos"]), w.top_k, w.sm_scale, out_dtype=torch.float32, want_lse=True,
                                workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    f = oracle.bf16_bits_to_f64
    _, ref_idx, ref_out, ref_lse = oracle.prefill(f(d["q_idx"]), d["w"].astype(np.float64), f(d["k_idx"]),
                                                  f(d["q"]), f(d["kv"]), pos, w.top_k, w.sm_scale)
    assert np.array_equal(host(idx), ref_idx)
    got = out_f64(out)
    assert np.abs(got - ref_out).max() <= 2e-3 * np.abs(ref_out).max()
    assert np.abs(host(lse) - ref_lse).max() < 2e-3
