"""The no-allocation DCP partial (sma_dcp_shard_partial_noalloc, scratch in
the library's static device array) against the workspace entry
(sma_dcp_shard_partial) on the same inputs: two calls in a row on one
stream, the second smaller, for bf16 rows, per-token FP8 rows and 656-byte
fp8_ds_mla rows.  Where both entries split a batch into the same number of
row slices the results are identical; where the static scratch holds fewer
slices they differ by the bf16 rounding of the softmax weights."""
import numpy as np
import pytest
import torch

import sparse_mla_attention_index_amd as sma
from sparse_mla_attention_index_amd import synth
from _gpuhelp import dev

pytestmark = pytest.mark.gpu

P, RANK, N_K = 8, 3, 24000


def _selection(n_q, top_k, seed):
    """Index lists as the top-k writes them: ascending global positions of
    each query's causal prefix, -1 padded; one query with an empty list and
    one whose tokens all sit on other ranks."""
    rng = np.random.default_rng(seed)
    idx = np.full((n_q, top_k), -1, dtype=np.int32)
    for i in range(n_q):
        p = int(rng.integers(top_k // 2, N_K))
        m = min(top_k, p + 1)
        idx[i, :m] = np.sort(rng.choice(p + 1, size=m, replace=False))
    idx[1, :] = -1
    idx[2, :] = -1
    idx[2, :4] = [0, 1, 2, 4]             # none on rank 3
    return idx


def _kv(kind):
    if kind == "bf16":
        x = synth.rows(synth.workload(2), "kv", 0, N_K)
        return (dev(np.ascontiguousarray(x[RANK::P])), None)
    w5 = synth.workload(5)
    if kind == "fp8":
        codes, scale = synth.rows(w5, "kv", 0, N_K)
        return (dev(np.ascontiguousarray(codes[RANK::P])), dev(np.ascontiguousarray(scale[RANK::P])))
    rows = synth.latent_rows_fp8_ds_mla(w5, 0, N_K)
    return (dev(np.ascontiguousarray(rows[RANK::P])), None)


@pytest.mark.parametrize("kind", ["bf16", "fp8", "fp8_ds_mla"])
def test_noalloc_matches_workspace_entry(kind):
    w = synth.workload(2)
    kv, kvs = _kv(kind)
    calls = [(64, 2048, 11), (5, 512, 12)]           # the second call is smaller
    inputs, res_na = [], []
    for n_q, top_k, seed in calls:
        q = dev(synth.rows(w, "q", 0, n_q))
        idx = dev(_selection(n_q, top_k, seed))
        out = torch.empty((n_q, 64, 512), dtype=torch.float32, device="cuda:0")
        lse = torch.empty((n_q, 64), dtype=torch.float32, device="cuda:0")
        inputs.append((q, idx))
        res_na.append((out, lse))
    # the two no-allocation calls back to back on the stream (outputs given)
    for (q, idx), (out, lse) in zip(inputs, res_na):
        sma.dcp_shard_partial_noalloc(RANK, P, q, kv, idx, w.sm_scale, kv_scale_local=kvs, out=out, lse=lse)
    res_ws = [sma.dcp_shard_partial(RANK, P, q, kv, idx, w.sm_scale, kv_scale_local=kvs) for q, idx in inputs]
    torch.cuda.synchronize()
    for c, ((o_na, l_na), (o_ws, l_ws)) in enumerate(zip(res_na, res_ws)):
        assert torch.isfinite(o_na).all(), c
        # queries with no token on the rank: 0 and -inf in both
        assert torch.equal(torch.isinf(l_na), torch.isinf(l_ws)), c
        assert torch.isinf(l_na[1]).all() and torch.isinf(l_na[2]).all() and (o_na[1:3] == 0).all(), c
        if c == 1:
            # 5 queries: the same slices either way, bit for bit
            assert torch.equal(o_na, o_ws) and torch.equal(l_na, l_ws), c
        else:
            # 64 queries: 7 slices fit the 64 MiB scratch beside the index
            # list, the full workspace takes 8.  The softmax weights enter PV
            # as bf16, rounded against each slice's own exponent reference,
            # so the outputs differ by that rounding (~2^-8 relative per
            # weight): held to the bf16 attention bar, 1e-2 of max|ref| (the
            # FP8 one is 3e-2); the LSE sums fp32 weights, fp32 summation
            # order only.
            scale = o_ws.abs().max().item()
            assert (o_na - o_ws).abs().max().item() <= 1e-2 * scale, c
            fin = torch.isfinite(l_ws)
            assert (l_na[fin] - l_ws[fin]).abs().max().item() <= 1e-4, c
