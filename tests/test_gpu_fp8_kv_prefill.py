"""GPU parity of sparse MLA over per-token FP8 latent rows at prefill batch
sizes (the FP8 rows gathered into LDS and widened to bf16 there, the row
scale on each row's logit and softmax weight), against the oracle on index
lists given to both sides.  The widening is exact (every e4m3 value is a
bf16 value); the weight PV takes, softmax weight times row scale, is
rounded to bf16 (2^-9 relative), so outputs are held to 1e-2 of max|ref|
for either output type (the FP8 bar is 3e-2), the LSE (fp32 weights) to
2e-3."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_index_amd as sma
from sparse_mla_attention_index_amd import synth
from _gpuhelp import dev, host, out_f64

pytestmark = pytest.mark.gpu
TAU = 1.0 / np.sqrt(192.0)


def _idx(n_q, n_k, top_k, seed):
    rng = np.random.default_rng(seed)
    idx = np.full((n_q, top_k), -1, dtype=np.int32)
    for i in range(n_q):
        m = int(min([top_k, 1, 33, top_k - 17, rng.integers(1, top_k + 1)][i % 5], n_k))
        idx[i, :m] = np.sort(rng.choice(n_k, m, replace=False))
    idx[1, 3] = n_k + 7              # past the context: skipped
    idx[2, :] = -1                   # empty selection
    idx[3, ::3] = -1                 # padding in the middle
    idx[4, : min(top_k, 96)] = -1    # the first tiles hold no valid row
    return idx


def _rows(n_k, seed, spread=False):
    """FP8 rows: the decode workload's quantised N(0,1) rows, or random codes
    (no NaN codes) with scales spread over six decades, some zero."""
    if not spread:
        return synth.rows(synth.workload(5), "kv", 0, n_k)
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, size=(n_k, 576)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x00      # drop the NaN codes
    scale = (10.0 ** rng.uniform(-3, 0, size=n_k)).astype(np.float32) * np.float32(1e-2)
    scale[::11] = 0.0
    return codes, scale


def _run(q, kv, idx, out_dtype, workspace=None):
    kvc, kvs = dev(kv)
    return sma.sparse_mla_prefill(dev(q), kvc, dev(idx), TAU, kv_scale=kvs, out_dtype=out_dtype, want_lse=True,
                                  workspace=workspace)


def _check(out, lse, q, kv, idx, rel):
    keep = np.where((idx >= 0) & (idx < kv[0].shape[0]), idx, -1)
    ref, ref_lse = oracle.sparse_mla(oracle.bf16_bits_to_f64(q), oracle.fp8_rows_to_f64(*kv), keep, TAU)
    got = out_f64(out)
    assert np.abs(got - ref).max() <= rel * np.abs(ref).max()
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(host(lse)), fin)
    assert np.abs(host(lse)[fin] - ref_lse[fin]).max() < 2e-3
    assert np.all(got[2] == 0)
    return got


@pytest.mark.parametrize("out_dtype,rel", [(torch.bfloat16, 1e-2), (torch.float32, 1e-2)])
@pytest.mark.parametrize("top_k", [2048, 100])
def test_fp8_rows_prefill_batch(out_dtype, rel, top_k):
    """300 queries (more than the CUs: no row slices, whatever the workspace)."""
    n_q, n_k = 300, 9000
    q = synth.rows(synth.workload(2), "q", 0, n_q)
    kv = _rows(n_k, 0)
    idx = _idx(n_q, n_k, top_k, 3)
    ws = torch.empty(max(1, sma.workspace_bytes(sma._lib.SMA_OP_SPARSE_MLA, n_q, n_k, top_k)), dtype=torch.uint8,
                     device="cuda:0")
    out, lse = _run(q, kv, idx, out_dtype, ws)
    _check(out, lse, q, kv, idx, rel)


def test_fp8_rows_spread_and_zero_scales():
    n_q, n_k, top_k = 260, 4000, 2048
    q = synth.rows(synth.workload(2), "q", 0, n_q)
    kv = _rows(n_k, 5, spread=True)
    idx = _idx(n_q, n_k, top_k, 7)
    out, lse = _run(q, kv, idx, torch.float32)
    _check(out, lse, q, kv, idx, 1e-2)


def test_fp8_rows_logits_rising_far_above_first_tile():
    """Rows whose logits pass the first valid tile's maximum by far more
    than the fixed-reference range: the query is swept again."""
    rng = np.random.default_rng(21)
    n_q, n_k, top_k = 260, 400, 256
    q = np.abs(rng.standard_normal((n_q, 64, 576)).astype(np.float32)) * np.float32(0.1) + np.float32(0.05)
    codes = rng.integers(1, 0x70, size=(n_k, 576)).astype(np.uint8)   # positive e4m3 values
    scale = np.full(n_k, 1e-3, dtype=np.float32)
    scale[300:] = 0.5                                                  # these rows: logits far above the rest
    idx = np.stack([np.sort(rng.choice(n_k, top_k, replace=False)) for _ in range(n_q)]).astype(np.int32)
    idx[:, :40] = np.arange(40)
    idx = np.sort(idx, axis=1)
    qb = synth.to_bf16_bits(q)
    kv = (codes, scale)
    kvc, kvs = dev(kv)
    out, lse = sma.sparse_mla_prefill(dev(qb), kvc, dev(idx), TAU, kv_scale=kvs, out_dtype=torch.float32,
                                      want_lse=True)
    ref, ref_lse = oracle.sparse_mla(oracle.bf16_bits_to_f64(qb), oracle.fp8_rows_to_f64(codes, scale), idx, TAU)
    got = out_f64(out)
    assert np.all(np.isfinite(got))
    assert np.abs(got - ref).max() <= 1e-2 * np.abs(ref).max()
    assert np.abs(host(lse) - ref_lse).max() <= 1e-3 * np.abs(ref_lse).max()


def test_fp8_rows_agree_with_split_kernel_and_deterministic():
    """A 40-query batch without workspace (this kernel) against the same
    batch with the workspace (rows split into slices, the decode kernel);
    the first run twice, bit for bit."""
    n_q, n_k, top_k = 40, 6000, 2048
    q = synth.rows(synth.workload(2), "q", 0, n_q)
    kv = _rows(n_k, 0)
    idx = _idx(n_q, n_k, top_k, 11)
    a, la = _run(q, kv, idx, torch.float32)
    b, lb = _run(q, kv, idx, torch.float32)
    ws = torch.empty(sma.workspace_bytes(sma._lib.SMA_OP_SPARSE_MLA, n_q, n_k, top_k), dtype=torch.uint8,
                     device="cuda:0")
    c, lc = _run(q, kv, idx, torch.float32, ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
    got = _check(a, la, q, kv, idx, 1e-2)
    assert np.abs(out_f64(c) - got).max() <= 1e-2 * np.abs(got).max()
