"""Edge cases of sma_sparse_mla_prefill for every KV row format (bf16,
per-token FP8, 656-byte fp8_ds_mla), with and without the workspace that
lets a small batch split its rows (up to the sixteen slices the merge
takes): top_k of 1 and around the 32-row tile,
contexts of one and two rows, a query whose only valid entry is the last
slot, a fully padded query, repeated entries (each counts, as the oracle
takes the list as given), and a single query.  Against the oracle, 1e-2 of
max|ref| for bf16 rows and 3e-2 for FP8 rows, LSE within 5e-3."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_index_amd as sma
from sparse_mla_attention_index_amd import _lib, synth
from _gpuhelp import dev, host, out_f64

pytestmark = pytest.mark.gpu
TAU = 1.0 / np.sqrt(192.0)


def _kv(fmt, n_k):
    """(device args for the call, float64 rows for the oracle)."""
    if fmt == "bf16":
        rows = synth.rows(synth.workload(2), "kv", 0, n_k)
        return (dev(rows), None), oracle.bf16_bits_to_f64(rows)
    if fmt == "fp8":
        codes, scale = synth.rows(synth.workload(5), "kv", 0, n_k)
        return dev((codes, scale)), oracle.fp8_rows_to_f64(codes, scale)
    rng = np.random.default_rng(n_k)
    rows = synth.to_fp8_ds_mla_rows(rng.standard_normal((n_k, 576)).astype(np.float32))
    return (dev(rows), None), oracle.fp8_ds_mla_rows_to_f64(rows)


def _check(q, kv_args, kv64, idx, fmt, split):
    n_q, top_k = idx.shape
    n_k = kv64.shape[0]
    ws = None
    if split:
        nb = sma.workspace_bytes(_lib.SMA_OP_SPARSE_MLA, n_q, n_k, top_k)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda:0")
    out, lse = sma.sparse_mla_prefill(dev(q), kv_args[0], dev(idx), TAU, kv_scale=kv_args[1],
                                      out_dtype=torch.float32, want_lse=True, workspace=ws)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.sparse_mla(oracle.bf16_bits_to_f64(q), kv64, np.where(idx < n_k, idx, -1), TAU)
    got, gl = out_f64(out), host(lse)
    tol = 1e-2 if fmt == "bf16" else 3e-2
    assert np.abs(got - ref).max() <= tol * max(np.abs(ref).max(), 1e-30)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(gl), fin)
    assert np.abs(gl[fin] - ref_lse[fin]).max(initial=0.0) < 5e-3
    empty = ~np.any((idx >= 0) & (idx < n_k), axis=1)
    assert np.all(got[empty] == 0)


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("fmt", ["bf16", "fp8", "fp8_ds_mla"])
@pytest.mark.parametrize("top_k", [1, 31, 32, 33, 64, 2047, 2048])   # 2048: sixteen row slices
def test_top_k_around_the_tile(fmt, split, top_k):
    n_q, n_k = 6, 3000
    rng = np.random.default_rng(top_k)
    q = synth.rows(synth.workload(2), "q", 0, n_q)
    kv_args, kv64 = _kv(fmt, n_k)
    idx = np.full((n_q, top_k), -1, dtype=np.int32)
    for i in range(n_q):
        m = [top_k, max(1, top_k // 2), 1, top_k, 0, top_k][i]
        idx[i, :m] = np.sort(rng.choice(n_k, m, replace=False)) if m else []
    idx[3, :] = -1
    idx[3, top_k - 1] = 17              # the only valid entry in the last slot
    _check(q, kv_args, kv64, idx, fmt, split)


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("fmt", ["bf16", "fp8", "fp8_ds_mla"])
def test_tiny_contexts_repeats_and_one_query(fmt, split):
    q = synth.rows(synth.workload(2), "q", 0, 3)
    for n_k in (1, 2):
        kv_args, kv64 = _kv(fmt, n_k)
        idx = np.array([[0, -1, -1], [n_k - 1, 0, n_k - 1], [-1, -1, -1]], dtype=np.int32)
        _check(q, kv_args, kv64, idx, fmt, split)
    kv_args, kv64 = _kv(fmt, 500)
    rng = np.random.default_rng(5)
    idx = rng.integers(0, 500, size=(1, 700)).astype(np.int32)   # one query, repeated rows
    idx[0, 650:] = -1
    _check(q[:1], kv_args, kv64, idx, fmt, split)
