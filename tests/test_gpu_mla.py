"""GPU parity of sma_sparse_mla_prefill against the oracle, on index lists
given to both sides (so the kernel's error is measured apart from the
selection's)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_index_amd as sma
from sparse_mla_attention_index_amd import synth
from _gpuhelp import dev, host, out_f64

pytestmark = pytest.mark.gpu
TAU = 1.0 / np.sqrt(192.0)


def _idx_lists(n_q, n_k, top_k, seed, invalid=False):
    rng = np.random.default_rng(seed)
    idx = np.full((n_q, top_k), -1, dtype=np.int32)
    for i in range(n_q):
        m = [top_k, 1, 17, top_k - 31, rng.integers(1, top_k + 1)][i % 5] if i % 7 else top_k
        m = int(min(m, n_k))
        idx[i, :m] = np.sort(rng.choice(n_k, m, replace=False))
    if invalid:
        idx[1, 3] = n_k + 5          # out of range: skipped
        idx[2, :] = -1               # empty set
        idx[3, ::2] = -1             # padding in the middle
        idx[5, :64] = -1             # leading padding: the first tiles hold no valid row
    return idx


def _inputs(w, n_q, n_k):
    q = synth.rows(w, "q", 0, n_q)
    kv = synth.rows(w, "kv", 0, n_k)
    return q, kv


def _ref(q, kv, idx, fp8=False):
    kvf = oracle.keys_f64(kv, fp8)
    keep = np.where((idx >= 0) & (idx < kvf.shape[0]), idx, -1)
    return oracle.sparse_mla(oracle.bf16_bits_to_f64(q), kvf, keep, TAU)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("top_k", [2048, 100])
def test_mla_bf16_kv(out_dtype, top_k):
    w = synth.workload(2)
    n_q, n_k = 40, 6000
    q, kv = _inputs(w, n_q, n_k)
    idx = _idx_lists(n_q, n_k, top_k, top_k, invalid=True)
    out, lse = sma.sparse_mla_prefill(dev(q), dev(kv), dev(idx), TAU, out_dtype=out_dtype, want_lse=True)
    ref, ref_lse = _ref(q, kv, idx)
    got = out_f64(out)
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    assert err <= 1e-2 * scale, (err, scale)
    if out_dtype == torch.float32:
        assert err <= 2e-3 * scale, (err, scale)
    gl = host(lse)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(gl), fin)
    assert np.abs(gl[fin] - ref_lse[fin]).max() < 2e-3
    assert np.all(got[2] == 0)


def test_mla_dense_causal_equivalence():
    """All causal tokens selected (top_k >= L): the kernel reproduces the
    oracle, which is pinned to dense causal attention."""
    w = synth.workload(1)
    L = 200
    q, kv = _inputs(w, L, L)
    idx = np.full((L, 256), -1, dtype=np.int32)
    for i in range(L):
        idx[i, : i + 1] = np.arange(i + 1)
    out, _ = sma.sparse_mla_prefill(dev(q), dev(kv), dev(idx), TAU, out_dtype=torch.float32)
    ref, _ = _ref(q, kv, idx)
    assert np.abs(out_f64(out) - ref).max() <= 2e-3 * np.abs(ref).max()


def test_mla_fp8_kv():
    w = synth.workload(5)
    n_q, n_k, top_k = 24, 5000, 2048
    q = synth.rows(synth.workload(2), "q", 0, n_q)
    kv = synth.rows(w, "kv", 0, n_k)
    idx = _idx_lists(n_q, n_k, top_k, 5)
    kvc, kvs = dev(kv)
    out, lse = sma.sparse_mla_prefill(dev(q), kvc, dev(idx), TAU, kv_scale=kvs, out_dtype=torch.bfloat16,
                                      want_lse=True)
    ref, ref_lse = _ref(q, kv, idx, fp8=True)
    got = out_f64(out)
    assert np.abs(got - ref).max() <= 3e-2 * np.abs(ref).max()
    assert np.abs(host(lse) - ref_lse).max() < 5e-3


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_mla_fp8_kv_split_rows(out_dtype):
    """A small FP8 batch given the workspace splits each query's rows into
    slices merged by log-sum-exp; same tolerance as the unsplit kernel,
    including empty lists and padding in the middle."""
    w = synth.workload(5)
    n_q, n_k, top_k = 12, 7000, 2048
    q = synth.rows(synth.workload(2), "q", 0, n_q)
    kv = synth.rows(w, "kv", 0, n_k)
    idx = _idx_lists(n_q, n_k, top_k, 21, invalid=True)
    kvc, kvs = dev(kv)
    nb = sma.workspace_bytes(sma._lib.SMA_OP_SPARSE_MLA, n_q, n_k, top_k)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out, lse = sma.sparse_mla_prefill(dev(q), kvc, dev(idx), TAU, kv_scale=kvs, out_dtype=out_dtype,
                                      want_lse=True, workspace=ws)
    ref, ref_lse = _ref(q, kv, idx, fp8=True)
    got = out_f64(out)
    assert np.abs(got - ref).max() <= 3e-2 * np.abs(ref).max()
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(host(lse)), fin)
    assert np.abs(host(lse)[fin] - ref_lse[fin]).max() < 5e-3
    assert np.all(got[2] == 0)   # the empty list
    # against the unsplit kernel on the same inputs
    one, _ = sma.sparse_mla_prefill(dev(q), kvc, dev(idx), TAU, kv_scale=kvs, out_dtype=out_dtype)
    assert np.abs(out_f64(one) - got).max() <= 1e-2 * np.abs(ref).max()


def test_mla_deterministic():
    w = synth.workload(2)
    q, kv = _inputs(w, 16, 3000)
    idx = _idx_lists(16, 3000, 2048, 9)
    a, _ = sma.sparse_mla_prefill(dev(q), dev(kv), dev(idx), TAU)
    b, _ = sma.sparse_mla_prefill(dev(q), dev(kv), dev(idx), TAU)
    assert torch.equal(a, b)


def test_mla_logits_rising_far_above_first_tile():
    """Later selected rows whose logits exceed the first tile's maximum by
    far more than the fixed-reference range (the kernel then sweeps the
    query again with the exact maximum)."""
    rng = np.random.default_rng(21)
    n_q, n_k, top_k = 6, 400, 256
    q = (rng.standard_normal((n_q, 64, 576)) * 0.1).astype(np.float32)
    kv = (rng.standard_normal((n_k, 576)) * 0.1).astype(np.float32)
    q[:, :, :] = np.abs(q) + 0.05               # positive, so large rows give large logits
    kv[300:] = np.abs(kv[300:]) * 100 + 5.0      # rows 300.. carry logits ~100 log2 units above the rest
    idx = np.stack([np.sort(rng.choice(n_k, top_k, replace=False)) for _ in range(n_q)]).astype(np.int32)
    idx[:, :40] = np.arange(40)                  # the first tile holds small rows only
    idx = np.sort(idx, axis=1)
    qb, kvb = synth.to_bf16_bits(q), synth.to_bf16_bits(kv)
    out, lse = sma.sparse_mla_prefill(dev(qb), dev(kvb), dev(idx), TAU, out_dtype=torch.float32, want_lse=True)
    ref, ref_lse = _ref(qb, kvb, idx)
    got = out_f64(out)
    assert np.all(np.isfinite(got))
    assert np.abs(got - ref).max() <= 2e-3 * np.abs(ref).max()
    assert np.abs(host(lse) - ref_lse).max() <= 1e-3 * np.abs(ref_lse).max()
