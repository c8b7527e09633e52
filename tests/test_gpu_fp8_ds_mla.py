"""GPU parity of sparse MLA over FlashMLA's 656-byte fp8_ds_mla latent rows
(512 e4m3 codes, four fp32 scales of 128 dims each, 64 bf16 rope dims),
against the oracle on the decoded rows, for the whole and the split kernel,
the composed prefill and the DCP shard partials."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_index_amd as sma
from sparse_mla_attention_index_amd import synth
from _gpuhelp import dev, host, out_f64

pytestmark = pytest.mark.gpu
TAU = 1.0 / np.sqrt(192.0)


def _ds_rows(n, seed):
    """Latent rows whose four 128-dim blocks and rope part have different
    magnitudes, so each block gets its own scale."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 576)).astype(np.float32) * 0.1
    for b, f in enumerate([0.25, 1.0, 4.0, 0.5]):
        x[:, 128 * b:128 * (b + 1)] *= f
    x[:, 512:] *= 2.0
    x[7, 256:384] = 0.0                 # an all-zero block: scale 0
    return synth.to_fp8_ds_mla_rows(x)


def _idx_lists(n_q, n_k, top_k, seed):
    rng = np.random.default_rng(seed)
    idx = np.full((n_q, top_k), -1, dtype=np.int32)
    for i in range(n_q):
        m = [top_k, 1, 33, top_k - 7, int(rng.integers(1, top_k + 1))][i % 5]
        m = min(m, n_k)
        idx[i, :m] = np.sort(rng.choice(n_k, m, replace=False))
    idx[1, 0] = n_k + 9      # out of range: skipped
    idx[2, :] = -1           # empty set
    idx[3, ::3] = -1         # padding in the middle
    if n_q > 4:
        idx[4, : min(top_k, 96)] = -1   # the first tiles hold no valid row
    return idx


def _ref(q, rows, idx):
    kvf = oracle.fp8_ds_mla_rows_to_f64(rows)
    keep = np.where((idx >= 0) & (idx < kvf.shape[0]), idx, -1)
    return oracle.sparse_mla(oracle.bf16_bits_to_f64(q), kvf, keep, TAU)


def _check(out, lse, ref, ref_lse, empty_row=2):
    got = out_f64(out)
    assert np.abs(got - ref).max() <= 3e-2 * np.abs(ref).max()
    gl = host(lse)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(gl), fin)
    assert np.abs(gl[fin] - ref_lse[fin]).max() < 5e-3
    assert np.all(got[empty_row] == 0)
    return got


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("top_k", [2048, 100])
def test_mla_fp8_ds_mla(out_dtype, top_k):
    n_q, n_k = 300, 6000     # more queries than CUs: the unsplit kernel
    rows = _ds_rows(n_k, top_k)
    q = synth.rows(synth.workload(2), "q", 0, n_q)
    idx = _idx_lists(n_q, n_k, top_k, top_k + 1)
    out, lse = sma.sparse_mla_prefill(dev(q), dev(rows), dev(idx), TAU, out_dtype=out_dtype, want_lse=True)
    ref, ref_lse = _ref(q, rows, idx)
    _check(out, lse, ref, ref_lse)


def test_mla_fp8_ds_mla_split_rows_and_determinism():
    """A small batch with the workspace splits each query's rows into
    slices merged by log-sum-exp; the same inputs twice give the same bits."""
    n_q, n_k, top_k = 12, 7000, 2048
    rows = _ds_rows(n_k, 31)
    q = synth.rows(synth.workload(2), "q", 0, n_q)
    idx = _idx_lists(n_q, n_k, top_k, 32)
    nb = sma.workspace_bytes(sma._lib.SMA_OP_SPARSE_MLA, n_q, n_k, top_k)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    out, lse = sma.sparse_mla_prefill(dev(q), dev(rows), dev(idx), TAU, want_lse=True, workspace=ws)
    ref, ref_lse = _ref(q, rows, idx)
    _check(out, lse, ref, ref_lse)
    out2, lse2 = sma.sparse_mla_prefill(dev(q), dev(rows), dev(idx), TAU, want_lse=True, workspace=ws)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_fp8_ds_mla_matches_per_row_format_when_scales_agree():
    """Rows whose four block scales equal one per-row scale and whose rope
    values are those codes' values: the 656-byte format and the 576-code
    per-row format describe the same latent, and the two kernels agree."""
    w = synth.workload(5)
    n_q, n_k, top_k = 300, 3000, 512
    codes, scale = synth.rows(w, "kv", 0, n_k)
    scale = np.exp2(np.round(np.log2(scale))).astype(np.float32)   # powers of two: code x scale exact in bf16
    vals = oracle.fp8_rows_to_f64(codes, scale)
    rows = np.zeros((n_k, 656), np.uint8)
    rows[:, :512] = codes[:, :512]
    rows[:, 512:528] = np.repeat(scale.astype("<f4")[:, None], 4, axis=1).view(np.uint8)
    rope = synth.to_bf16_bits(vals[:, 512:].astype(np.float32))
    assert np.array_equal(oracle.bf16_bits_to_f64(rope), vals[:, 512:])   # e4m3 x scale with few bits: exact
    rows[:, 528:] = rope.astype("<u2").view(np.uint8)
    assert np.array_equal(oracle.fp8_ds_mla_rows_to_f64(rows), vals)
    q = synth.rows(synth.workload(2), "q", 0, n_q)
    idx = _idx_lists(n_q, n_k, top_k, 41)
    kvc, kvs = dev((codes, scale))
    a, la = sma.sparse_mla_prefill(dev(q), kvc, dev(idx), TAU, kv_scale=kvs, out_dtype=torch.float32, want_lse=True)
    b, lb = sma.sparse_mla_prefill(dev(q), dev(rows), dev(idx), TAU, out_dtype=torch.float32, want_lse=True)
    ref, _ = _ref(q, rows, idx)
    assert np.abs(out_f64(a) - out_f64(b)).max() <= 1e-2 * np.abs(ref).max()
    fin = torch.isfinite(la)
    assert torch.equal(fin, torch.isfinite(lb)) and float((la[fin] - lb[fin]).abs().max()) < 1e-3


def test_prefill_and_dcp_with_fp8_ds_mla_rows():
    """The composed prefill takes the 656-byte rows as its KV (index lists
    equal the bf16-KV run's, the indexer being unchanged), and DCP shards of
    those rows merge to the unsharded attention."""
    w = synth.workload(2)
    n = 900
    pos = np.arange(n, dtype=np.int32)
    q_idx, wt, k_idx = (synth.rows(w, "q_idx", 0, n), synth.rows(w, "w", 0, n), synth.rows(w, "k_idx", 0, n))
    q = synth.rows(w, "q", 0, n)
    rows = synth.latent_rows_fp8_ds_mla(w, 0, n)
    idx = torch.empty((n, 256), dtype=torch.int32, device="cuda:0")
    out, lse, _ = sma.prefill(dev(q_idx), dev(wt), dev(k_idx), dev(q), dev(rows), dev(pos), 256, TAU,
                              want_lse=True, idx_out=idx)
    idx_b = torch.empty_like(idx)
    sma.prefill(dev(q_idx), dev(wt), dev(k_idx), dev(q), dev(synth.rows(w, "kv", 0, n)), dev(pos), 256, TAU,
                idx_out=idx_b)
    assert torch.equal(idx, idx_b)
    gi = host(idx)
    rows_s = list(range(0, n, 37)) + [n - 1]
    ref, ref_lse = _ref(q[rows_s], rows, gi[rows_s])
    got = out_f64(out)[rows_s]
    assert np.abs(got - ref).max() <= 3e-2 * np.abs(ref).max()
    # DCP: 4 round-robin shards of the rows, partials merged by log-sum-exp
    P = 4
    parts = torch.empty((P, n, 64, 512), dtype=torch.float32, device="cuda:0")
    lses = torch.empty((P, n, 64), dtype=torch.float32, device="cuda:0")
    for r in range(P):
        sma.dcp_shard_partial(r, P, dev(q), dev(np.ascontiguousarray(rows[r::P])), idx, TAU, out=parts[r],
                              lse=lses[r])
    merged, _ = sma.lse_merge(parts, lses, out_dtype=torch.float32)
    full, _ = sma.sparse_mla_prefill(dev(q), dev(rows), idx, TAU, out_dtype=torch.float32)
    assert float((merged - full).abs().max()) <= 1e-2 * float(full.abs().max())


def test_fp8_ds_mla_logits_rising_far_above_first_tile():
    """Rows whose logits pass the first valid tile's maximum by far more than
    the fixed-reference range (the query is swept again), with the rope part
    carrying its share of the logit; both output types."""
    rng = np.random.default_rng(23)
    n_q, n_k, top_k = 260, 400, 256
    q = synth.to_bf16_bits(np.abs(rng.standard_normal((n_q, 64, 576)).astype(np.float32)) * np.float32(0.1)
                           + np.float32(0.05))
    x = np.abs(rng.standard_normal((n_k, 576)).astype(np.float32)) * np.float32(0.01)
    x[300:] += np.float32(12.0)                   # these rows: logits far above the rest
    rows = synth.to_fp8_ds_mla_rows(x)
    idx = np.stack([np.sort(rng.choice(n_k, top_k, replace=False)) for _ in range(n_q)]).astype(np.int32)
    idx[:, :40] = np.arange(40)
    idx = np.sort(idx, axis=1)
    ref, ref_lse = _ref(q, rows, idx)
    for out_dtype in (torch.float32, torch.bfloat16):
        out, lse = sma.sparse_mla_prefill(dev(q), dev(rows), dev(idx), TAU, out_dtype=out_dtype, want_lse=True)
        got = out_f64(out)
        assert np.all(np.isfinite(got))
        assert np.abs(got - ref).max() <= 3e-2 * np.abs(ref).max()
        # every code x block scale is rounded once to bf16 (2^-9 relative);
        # these rows' products all have one sign, so the logits (~70) carry
        # that relative error without cancellation: LSE within 2.5e-3 of it
        assert np.abs(host(lse) - ref_lse).max() <= 2.5e-3 * np.abs(ref_lse).max()
