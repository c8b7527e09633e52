"""GPU parity of one DCP rank's partial sparse MLA (sma_dcp_shard_partial)
and of the log-sum-exp merge (sma_lse_merge) against the oracle: each rank's
partial computed on its own shard, the merge of every rank's partials
against the unsharded attention (oracle and GPU), bf16 and FP8 shards,
queries with nothing on a rank, and the merge alone on random partials."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_index_amd as sma
from sparse_mla_attention_index_amd import synth
from _gpuhelp import dev, host, out_f64

pytestmark = pytest.mark.gpu
TAU = 1.0 / np.sqrt(192.0)


def _idx(n_q, n_k, top_k, seed, P):
    rng = np.random.default_rng(seed)
    idx = np.full((n_q, top_k), -1, dtype=np.int32)
    for i in range(n_q):
        m = int(min([top_k, 1, 37, top_k - 5, rng.integers(1, top_k + 1)][i % 5], n_k))
        idx[i, :m] = np.sort(rng.choice(n_k, m, replace=False))
    idx[4, :] = -1                                  # empty selection
    idx[6, :] = -1
    idx[6, :3] = [0, P, 2 * P]                      # every token on rank 0
    idx[7, 5] = n_k + 3                             # past the context: skipped
    return idx


def _shard(kv, r, P):
    if isinstance(kv, tuple):
        return tuple(np.ascontiguousarray(a[r::P]) for a in kv)
    return np.ascontiguousarray(kv[r::P])


def _close(got, ref, rel):
    scale = max(np.abs(ref).max(), 1e-30)
    err = np.abs(got - ref).max()
    assert err <= rel * scale, (err, scale)


def _lse_close(got, ref, tol):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin)
    if fin.any():
        assert np.abs(got[fin] - ref[fin]).max() < tol


def _run(P, fp8, n_q, n_k, top_k, seed, rel, ltol):
    w = synth.workload(5 if fp8 else 2)
    q = synth.rows(synth.workload(2), "q", 0, n_q)
    kv = synth.rows(w, "kv", 0, n_k)
    idx = _idx(n_q, n_k, top_k, seed, P)
    q64, kv64 = oracle.bf16_bits_to_f64(q), oracle.keys_f64(kv, fp8)
    keep = np.where(idx < n_k, idx, -1)
    parts, lses = [], []
    for r in range(P):
        sh = dev(_shard(kv, r, P))
        kvl, kvs = (sh if fp8 else (sh, None))
        o, l = sma.dcp_shard_partial(r, P, dev(q), kvl, dev(idx), TAU, kv_scale_local=kvs)
        ro, rl = oracle.dcp_shard_partial(r, P, q64, kv64, keep, TAU)
        _close(host(o).astype(np.float64), ro, rel)
        _lse_close(host(l), rl, ltol)
        assert np.all(host(o)[4] == 0)
        if r > 0:
            assert np.all(np.isneginf(host(l)[6]))      # rank r > 0 stores none of query 6's tokens
        parts.append(o)
        lses.append(l)
    out, lse = sma.lse_merge(torch.stack(parts).contiguous(), torch.stack(lses).contiguous(),
                             out_dtype=torch.float32, want_lse=True)
    ref, ref_lse = oracle.sparse_mla(q64, kv64, keep, TAU)
    _close(out_f64(out), ref, rel)
    _lse_close(host(lse), ref_lse, ltol)
    assert np.all(out_f64(out)[4] == 0)
    return q, kv, idx, out, ref


@pytest.mark.parametrize("P", [1, 3, 8])
def test_dcp_bf16_shards_merge_to_unsharded(P):
    q, kv, idx, out, ref = _run(P, False, 24, 6000, 2048, P, 2e-3, 2e-3)
    full, _ = sma.sparse_mla_prefill(dev(q), dev(kv), dev(idx), TAU, out_dtype=torch.float32)
    _close(out_f64(out), out_f64(full), 2e-3)


def test_dcp_fp8_shards_merge_to_unsharded():
    """FP8 shards of a decode-sized batch (each partial splits its rows
    across workgroups inside the library)."""
    q, kv, idx, out, ref = _run(8, True, 16, 9000, 2048, 31, 3e-2, 5e-3)
    kvc, kvs = dev(kv)
    full, _ = sma.sparse_mla_prefill(dev(q), kvc, dev(idx), TAU, kv_scale=kvs, out_dtype=torch.float32)
    _close(out_f64(out), out_f64(full), 1e-2)


@pytest.mark.parametrize("P", [5, 1, 4, 9, 64])   # the merge loads ranks four at a time; 64 is the maximum
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_lse_merge_random_partials(out_dtype, P):
    rng = np.random.default_rng(3 + P)
    n_q = 7
    parts = rng.standard_normal((P, n_q, 64, 512)).astype(np.float32)
    lses = (rng.standard_normal((P, n_q, 64)) * 4).astype(np.float32)
    lses[min(1, P - 1), 2, :] = -np.inf  # one empty partial
    lses[:, 3, 10] = -np.inf             # an all-empty (query, head)
    out, lse = sma.lse_merge(dev(parts), dev(lses), out_dtype=out_dtype, want_lse=True)
    ref, ref_lse = oracle.lse_merge(parts.astype(np.float64), lses.astype(np.float64))
    _close(out_f64(out), ref, 1e-5 if out_dtype == torch.float32 else 8e-3)
    _lse_close(host(lse), ref_lse, 1e-5)
    assert np.all(out_f64(out)[3, 10] == 0)


def test_dcp_deterministic():
    w = synth.workload(2)
    q = synth.rows(w, "q", 0, 8)
    kv = synth.rows(w, "kv", 0, 3000)
    idx = _idx(8, 3000, 512, 2, 4)
    a, la = sma.dcp_shard_partial(1, 4, dev(q), dev(_shard(kv, 1, 4)), dev(idx), TAU)
    b, lb = sma.dcp_shard_partial(1, 4, dev(q), dev(_shard(kv, 1, 4)), dev(idx), TAU)
    assert torch.equal(a, b) and torch.equal(la, lb)
