"""The release library under HIP graph capture.  Its calls launch kernels on
the caller's stream and nothing else (no allocation, no memset, no
synchronisation), so a decode-shaped step -- sma_prefill over FP8 keys and
FP8 latent rows (indexer, split top-k, split attention and merge) -- and a
DCP partial through the no-allocation entry can be captured into one graph.
The graph is replayed three times with the program's own work and
synchronisations between the replays, and every replay must give the eager
result bit for bit."""
import numpy as np
import pytest
import torch

import sparse_mla_attention_index_amd as sma
from sparse_mla_attention_index_amd import _lib, synth
from _gpuhelp import dev

pytestmark = pytest.mark.gpu


def _inputs(n_k, n_q):
    w = synth.workload(5)
    rng = np.random.default_rng(41)
    pos = np.sort(rng.integers(n_k - 50_000, n_k, size=n_q)).astype(np.int32)
    pos[0] = n_k - 1
    k_idx = synth.rows(w, "k_idx", 0, n_k)
    kv = synth.rows(w, "kv", 0, n_k)
    take = lambda t: np.concatenate([synth.rows(w, t, p, p + 1) for p in pos])
    return w, pos, dev(k_idx), dev(kv), dev(take("q_idx")), dev(take("w")), dev(take("q"))


def test_decode_step_graph_replays_match_eager():
    n_k, n_q = 200_000, 16
    w, pos, (kc, ks), (vc, vs), q_idx, wt, q = _inputs(n_k, n_q)
    q_pos = dev(pos)
    nb = sma.workspace_bytes(_lib.SMA_OP_PREFILL, n_q, n_k, w.top_k)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
    out = torch.empty((n_q, 64, 512), dtype=torch.bfloat16, device="cuda:0")
    idx = torch.empty((n_q, w.top_k), dtype=torch.int32, device="cuda:0")
    P, rank = 4, 1
    kv_l, ks_l = vc[rank::P].contiguous(), vs[rank::P].contiguous()
    part = torch.empty((n_q, 64, 512), dtype=torch.float32, device="cuda:0")
    lse = torch.empty((n_q, 64), dtype=torch.float32, device="cuda:0")

    def step():
        sma.prefill(q_idx, wt, kc, q, vc, q_pos, w.top_k, w.sm_scale, k_scale=ks, kv_scale=vs, out=out,
                    idx_out=idx, workspace=ws)
        sma.dcp_shard_partial_noalloc(rank, P, q, kv_l, idx, w.sm_scale, kv_scale_local=ks_l, out=part, lse=lse)

    step()   # eager: also takes the device's cached facts and the static scratch address
    torch.cuda.synchronize()
    ref = [t.clone() for t in (out, idx, part, lse)]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for replay in range(3):
        out.fill_(float("nan"))
        part.fill_(float("nan"))
        lse.fill_(float("nan"))
        idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((out, idx, part, lse), ref):
            assert torch.equal(got, want), replay
