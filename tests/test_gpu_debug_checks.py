"""The debug build (libsma_debug.so): on valid inputs it gives the release
build's results bit for bit, although every workspace (and the no-allocation
entry's static scratch) is filled with 0xFF bytes, fp32 NaN, before use, so
no kernel reads workspace it has not written; and it rejects, before any
other launch, the device-resident positions and index entries that the
release build clamps or skips (include/sma.h, conventions)."""
import numpy as np
import pytest
import torch

import sparse_mla_attention_index_amd as sma
from sparse_mla_attention_index_amd import _lib, synth
from _gpuhelp import dev

pytestmark = pytest.mark.gpu
TAU = 1.0 / np.sqrt(192.0)


def _both(fn):
    """fn() under the release build, then under the debug build."""
    a = fn()
    with _lib.debug_library():
        assert _lib.build_flags() == _lib.SMA_BUILD_DEBUG_CHECKS
        b = fn()
    torch.cuda.synchronize()
    return a, b


def _equal(a, b):
    if isinstance(a, (tuple, list)):
        assert len(a) == len(b)
        for x, y in zip(a, b):
            _equal(x, y)
    elif a is None:
        assert b is None
    else:
        assert torch.equal(a, b)


def _prefill_inputs(n, seed_rows=0):
    w = synth.workload(2)
    pos = np.arange(n, dtype=np.int32)
    return (dev(synth.rows(w, "q_idx", seed_rows, seed_rows + n)), dev(synth.rows(w, "w", 0, n)),
            dev(synth.rows(w, "k_idx", 0, n)), dev(synth.rows(w, "q", 0, n)), dev(synth.rows(w, "kv", 0, n)),
            dev(pos))


def test_same_bits_as_release_on_valid_inputs():
    n, top_k = 700, 256
    q_idx, wt, k_idx, q, kv, pos = _prefill_inputs(n)

    def composed():
        idx = torch.empty((n, top_k), dtype=torch.int32, device="cuda:0")
        out, lse, _ = sma.prefill(q_idx, wt, k_idx, q, kv, pos, top_k, TAU, want_lse=True, idx_out=idx)
        return out, lse, idx

    a, b = _both(composed)
    _equal(a, b)
    idx = a[2]
    # the attention alone on a small batch with its workspace (row slices
    # whose partials live in the workspace), bf16 and per-token FP8 rows
    sub = idx[:24].contiguous()
    nb = sma.workspace_bytes(_lib.SMA_OP_SPARSE_MLA, 24, n, top_k)
    assert nb > 0
    fp8_rows = dev(synth.rows(synth.workload(5), "kv", 0, n))
    for kv_t, kv_s in ((kv, None), fp8_rows):
        def attn():
            ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
            return sma.sparse_mla_prefill(q[:24].contiguous(), kv_t, sub, TAU, kv_scale=kv_s, want_lse=True,
                                          workspace=ws)
        _equal(*_both(attn))

    # top-k on scores with a NaN-filled split workspace, and a DCP partial
    scores = torch.randn((8, 70000), device="cuda:0")
    qp = torch.full((8,), 69999, dtype=torch.int32, device="cuda:0")
    _equal(*_both(lambda: sma.topk_select(scores, qp, 2048)))

    def dcp():
        r = sma.dcp_shard_partial(1, 3, q[:40].contiguous(), kv[1::3].contiguous(), idx[:40].contiguous(), TAU)
        s = sma.dcp_shard_partial_noalloc(1, 3, q[:40].contiguous(), kv[1::3].contiguous(), idx[:40].contiguous(),
                                          TAU)
        return r, s

    _equal(*_both(dcp))


def test_rejects_out_of_range_index_entries():
    n, n_q, top_k = 500, 40, 64
    _, _, _, q, kv, _ = _prefill_inputs(n)
    rng = np.random.default_rng(5)
    idx = np.sort(rng.integers(0, n, size=(n_q, top_k)), axis=1).astype(np.int32)
    for bad, where in ((n + 3, (7, 11)), (-5, (39, 63))):
        wrong = idx.copy()
        wrong[where] = bad
        out = torch.full((n_q, 64, 512), 7.0, dtype=torch.float32, device="cuda:0")
        with _lib.debug_library():
            with pytest.raises(_lib.SmaError) as ei:
                sma.sparse_mla_prefill(q[:n_q].contiguous(), kv, dev(wrong), TAU, out=out)
        assert ei.value.status == -1
        assert f"idx[{where[0] * top_k + where[1]}] = {bad}" in str(ei.value)
        torch.cuda.synchronize()
        assert bool((out == 7.0).all())          # nothing launched
    # the release build skips such entries (documented), so it runs
    wrong = idx.copy()
    wrong[7, 11] = n + 3
    sma.sparse_mla_prefill(q[:n_q].contiguous(), kv, dev(wrong), TAU)
    # a DCP shard's list holds global positions: only entries below -1 are out of range
    wrong = idx.copy()
    wrong[2, 5] = -2
    with _lib.debug_library():
        with pytest.raises(_lib.SmaError, match=r"idx\[133\] = -2"):
            sma.dcp_shard_partial(0, 2, q[:n_q].contiguous(), kv[0::2].contiguous(), dev(wrong), TAU)
        big = idx.copy()
        big[0, 0] = 10 * n                       # a global position past the shard: kept as valid input
        sma.dcp_shard_partial(0, 2, q[:n_q].contiguous(), kv[0::2].contiguous(), dev(big), TAU)
    torch.cuda.synchronize()


def test_rejects_out_of_range_positions():
    n = 300
    q_idx, wt, k_idx, q, kv, pos = _prefill_inputs(n)
    for bad in (n, -2):
        p = pos.clone()
        p[17] = bad
        scores = torch.full((n, n), 3.0, dtype=torch.float32, device="cuda:0")
        with _lib.debug_library():
            with pytest.raises(_lib.SmaError, match=rf"q_pos\[17\] = {bad}"):
                sma.index_scores(q_idx, wt, k_idx, p, scores=scores)
            with pytest.raises(_lib.SmaError, match=rf"q_pos\[17\] = {bad}"):
                sma.topk_select(scores, p, 64)
            with pytest.raises(_lib.SmaError, match=rf"q_pos\[17\] = {bad}"):
                sma.prefill(q_idx, wt, k_idx, q, kv, p, 64, TAU)
        torch.cuda.synchronize()
        assert bool((scores == 3.0).all())       # nothing launched
