"""The C ABI from plain C: tests/c_client/prefill_client (built by
build() with the host C compiler against include/sma.h, the HIP runtime's
C API and libsma.so, no Python or torch) runs sma_prefill on the tiny
integer workload (L = 512, top_k = 128, 8 x 64 indexer) in a process of its
own.  Its index lists must equal the oracle's exactly (the integer inputs
make every score exact), its output must be within 1e-2 of max|ref|, and
both must equal, bit for bit, what the Python binding gets from the same
library on the same inputs."""
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_index_amd as sma
from sparse_mla_attention_index_amd import synth
from _gpuhelp import dev

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "tests", "c_client", "prefill_client")


def test_c_client_prefill_matches_oracle_and_binding(tmp_path):
    assert os.path.exists(CLIENT), "tests/c_client/prefill_client is built by __graft_entry__.build()"
    w = synth.workload(1)
    n = w.n_keys
    pos = synth.query_positions(w)
    qi, wt, ki = synth.rows(w, "q_idx", 0, n), synth.rows(w, "w", 0, n), synth.rows(w, "k_idx", 0, n)
    q, kv = synth.rows(w, "q", 0, n), synth.rows(w, "kv", 0, n)
    with open(tmp_path / "meta.txt", "w") as f:
        # nine significant digits carry the fp32 scale exactly, as the binding passes it
        f.write(f"{n} {n} {w.h_idx} {w.d_idx} {w.top_k} {float(np.float32(w.sm_scale)):.9g}\n")
    for name, arr in (("q_idx", qi), ("w", wt), ("k_idx", ki), ("q", q), ("kv", kv), ("pos", pos)):
        np.ascontiguousarray(arr).tofile(tmp_path / f"{name}.bin")
    print(f"c client: L={n} top_k={w.top_k}", flush=True)
    r = subprocess.run([CLIENT, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    got_idx = np.fromfile(tmp_path / "idx.bin", dtype=np.int32).reshape(n, w.top_k)
    got_out = np.fromfile(tmp_path / "out.bin", dtype=np.float32).reshape(n, 64, 512)
    got_lse = np.fromfile(tmp_path / "lse.bin", dtype=np.float32).reshape(n, 64)

    f = oracle.bf16_bits_to_f64
    _, ref_idx, ref_out, ref_lse = oracle.prefill(f(qi), wt.astype(np.float64), f(ki), f(q), f(kv), pos,
                                                  w.top_k, w.sm_scale)
    assert np.array_equal(got_idx, ref_idx)
    assert np.abs(got_out - ref_out).max() <= 1e-2 * np.abs(ref_out).max()
    assert np.abs(got_lse - ref_lse).max() < 5e-3

    idx = torch.empty((n, w.top_k), dtype=torch.int32, device="cuda:0")
    out, lse, _ = sma.prefill(dev(qi), dev(wt), dev(ki), dev(q), dev(kv), dev(pos), w.top_k, w.sm_scale,
                              out_dtype=torch.float32, want_lse=True, idx_out=idx)
    torch.cuda.synchronize()
    assert np.array_equal(idx.cpu().numpy(), got_idx)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), got_out.view(np.uint32))
    assert np.array_equal(lse.cpu().numpy().view(np.uint32), got_lse.view(np.uint32))
