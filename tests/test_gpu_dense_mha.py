"""GPU parity of the dense MHA prefill (sma_dense_mha_prefill): the path for
prompts that fit inside top-k (GLM-5.3 part 2, "Essayez-le"; DeepSeek
multi-node page, "Travaux futurs").  Against the oracle's
dense_mha_prefill, and against the GPU's own absorbed sparse path (absorb_q
-> sparse MLA over every causal token -> project_out), which computes the
same attention.  Tolerance: 1e-2 of max|ref| for the outputs (the bf16
attention bar; the expanded keys and values and the softmax weights are
bf16 operands), 2e-3 for the LSE."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_index_amd as sma
from sparse_mla_attention_index_amd import synth
from _gpuhelp import dev, host, out_f64

pytestmark = pytest.mark.gpu
TAU = 1.0 / np.sqrt(192.0)


def _inputs(n_k, n_q, seed):
    """bf16 storage (uint16 bits): q [n_q, 64, 192] ~ 0.1 N(0,1) (no-rope
    dims then rope dims), the 16K workload's latent rows [n_k, 576],
    W_UK / W_UV [64, 128, 512] ~ 0.05 N(0,1)."""
    rng = np.random.default_rng(seed)
    q = synth.to_bf16_bits(rng.standard_normal((n_q, 64, 192), dtype=np.float32) * np.float32(0.1))
    kv = synth.rows(synth.workload(2), "kv", 0, n_k)
    w_uk = synth.to_bf16_bits(rng.standard_normal((64, 128, 512), dtype=np.float32) * np.float32(0.05))
    w_uv = synth.to_bf16_bits(rng.standard_normal((64, 128, 512), dtype=np.float32) * np.float32(0.05))
    return q, kv, w_uk, w_uv


def _oracle(q, kv, w_uk, w_uv, pos):
    f = oracle.bf16_bits_to_f64
    return oracle.dense_mha_prefill(f(q), f(kv), f(w_uk), f(w_uv), pos, TAU)


def _close(got, ref, rel=1e-2):
    scale = np.abs(ref).max()
    err = np.abs(got - ref).max()
    assert err <= rel * scale, f"max err {err:.3e} > {rel} * {scale:.3e}"


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_prompt_matches_oracle(out_dtype):
    """A 512-token prompt (several 128-query blocks and 32-key tiles),
    positions 0..511."""
    L = 512
    q, kv, w_uk, w_uv = _inputs(L, L, 1)
    pos = np.arange(L, dtype=np.int32)
    out, lse = sma.dense_mha_prefill(dev(q), dev(kv), dev(w_uk), dev(w_uv), dev(pos), TAU, out_dtype=out_dtype,
                                     want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = _oracle(q, kv, w_uk, w_uv, pos)
    _close(out_f64(out), ref)
    assert np.abs(host(lse) - ref_lse).max() < 2e-3


def test_ragged_scattered_positions():
    """1,000 keys (a ragged last tile), 300 queries (a ragged last block) at
    scattered positions: both ends of the prompt, out-of-order rows, an empty
    prefix (-1) and positions clamped to n_k-1."""
    n_k, n_q = 1000, 300
    q, kv, w_uk, w_uv = _inputs(n_k, n_q, 2)
    rng = np.random.default_rng(3)
    pos = rng.integers(0, n_k, size=n_q).astype(np.int32)
    pos[:6] = [0, n_k - 1, -1, 5000, 31, 32]
    out, lse = sma.dense_mha_prefill(dev(q), dev(kv), dev(w_uk), dev(w_uv), dev(pos), TAU, out_dtype=torch.float32,
                                     want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = _oracle(q, kv, w_uk, w_uv, np.clip(pos, -1, n_k - 1))
    got = out_f64(out)
    assert np.all(got[2] == 0) and np.all(np.isneginf(host(lse)[2]))
    _close(got, ref)
    fin = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(host(lse)), fin)
    assert np.abs(host(lse)[fin] - ref_lse[fin]).max() < 2e-3


def test_equals_absorbed_sparse_path_at_top_k():
    """A 2,048-token prompt (the top-k): the dense MHA path against the
    forced-MQA path on the GPU (absorb_q, sparse MLA over every causal token,
    project_out), and both against the oracle on sampled rows."""
    L = 2048
    q, kv, w_uk, w_uv = _inputs(L, L, 4)
    pos = np.arange(L, dtype=np.int32)
    qd, kvd, wk, wv = dev(q), dev(kv), dev(w_uk), dev(w_uv)
    out, lse = sma.dense_mha_prefill(qd, kvd, wk, wv, dev(pos), TAU, out_dtype=torch.float32, want_lse=True)
    # the absorbed path: q_abs = [W_UK^T q_nope, q_rope], every causal token selected
    q_abs = torch.empty((L, 64, 576), dtype=torch.int16, device="cuda:0")
    q_abs[:, :, 512:] = qd[:, :, 128:]
    sma.absorb_q(qd[:, :, :128].contiguous(), wk, out=q_abs)
    idx = np.full((L, L), -1, dtype=np.int32)
    for i in range(L):
        idx[i, : i + 1] = np.arange(i + 1)
    o_lat, lse_s = sma.sparse_mla_prefill(q_abs, kvd, dev(idx), TAU, out_dtype=torch.bfloat16, want_lse=True)
    o_mqa = sma.project_out(o_lat, wv)
    torch.cuda.synchronize()
    got = out_f64(out)
    _close(out_f64(o_mqa), got, 2e-2)     # two bf16 roundings more on the absorbed side (q_abs, o_lat)
    assert np.abs(host(lse) - host(lse_s)).max() < 5e-3
    rows = np.array([0, 1, 31, 32, 127, 128, 1000, 2046, 2047])
    ref, ref_lse = _oracle(q[rows], kv, w_uk, w_uv, pos[rows])
    _close(got[rows], ref)
    assert np.abs(host(lse)[rows] - ref_lse).max() < 2e-3


def test_deterministic():
    q, kv, w_uk, w_uv = _inputs(700, 700, 5)
    pos = np.arange(700, dtype=np.int32)
    a = sma.dense_mha_prefill(dev(q), dev(kv), dev(w_uk), dev(w_uv), dev(pos), TAU, want_lse=True)
    b = sma.dense_mha_prefill(dev(q), dev(kv), dev(w_uk), dev(w_uv), dev(pos), TAU, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
