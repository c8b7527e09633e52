"""GPU parity of sma_index_scores against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_index_amd as sma
from sparse_mla_attention_index_amd import synth
from _gpuhelp import dev, host

pytestmark = pytest.mark.gpu


def _run(q_idx, w, k, pos, k_scale=None, ld=None, fill=np.nan):
    n_q, n_k = q_idx.shape[0], (k[0] if isinstance(k, tuple) else k).shape[0]
    ld = n_k if ld is None else ld
    scores = torch.full((n_q, ld), fill, dtype=torch.float32, device="cuda:0")
    kk = dev(k)
    if isinstance(kk, tuple):
        kk, ks = kk
    else:
        ks = None
    sma.index_scores(dev(q_idx), dev(w), kk, dev(pos), k_scale=ks, scores=scores)
    torch.cuda.synchronize()
    return host(scores)


def _oracle(q_idx, w, k, pos, fp8=False):
    return oracle.index_scores(oracle.bf16_bits_to_f64(q_idx), w.astype(np.float64),
                               oracle.keys_f64(k, fp8), pos)


def test_tiny_workload_exact():
    """Integer q_I/k_I and w = k/16: every score is exact in fp32."""
    w = synth.workload(1)
    pos = synth.query_positions(w)
    q = synth.rows(w, "q_idx", 0, w.n_keys)
    wt = synth.rows(w, "w", 0, w.n_keys)
    k = synth.rows(w, "k_idx", 0, w.n_keys)
    got = _run(q, wt, k, pos)
    ref = _oracle(q, wt, k, pos)
    for i, p in enumerate(pos):
        assert np.array_equal(got[i, : p + 1].astype(np.float64), ref[i]), i
        assert np.all(np.isnan(got[i, p + 1:]))


def _int_inputs(seed, n, h, d):
    rng = np.random.default_rng(seed)
    q = synth.to_bf16_bits(rng.integers(-3, 4, size=(n, h, d)).astype(np.float32))
    k = synth.to_bf16_bits(rng.integers(-3, 4, size=(n, d)).astype(np.float32))
    wt = (rng.integers(0, 17, size=(n, h)) / 16).astype(np.float32)
    return q, wt, k


@pytest.mark.parametrize("h,d", [(64, 128), (64, 64), (32, 128), (16, 64), (8, 128)])
def test_integer_exact_all_shapes(h, d):
    n = 1000 + 37   # several tiles and a ragged tail
    q, wt, k = _int_inputs(h * d, n, h, d)
    pos = np.arange(n, dtype=np.int32)
    got = _run(q, wt, k, pos)
    ref = _oracle(q, wt, k, pos)
    for i in range(0, n, 7):
        assert np.array_equal(got[i, : i + 1].astype(np.float64), ref[i]), i


def test_normal_inputs_tolerance():
    w = synth.workload(2)
    n = 2500
    q = synth.rows(w, "q_idx", 0, n)
    wt = synth.rows(w, "w", 0, n)
    k = synth.rows(w, "k_idx", 0, n)
    pos = np.arange(n, dtype=np.int32)
    got = _run(q, wt, k, pos)
    ref = _oracle(q, wt, k, pos)
    worst = 0.0
    for i in range(0, n, 11):
        r = ref[i]
        err = np.abs(got[i, : i + 1] - r).max() / np.abs(r).max()
        worst = max(worst, err)
    assert worst < 1e-5, worst


def test_shared_weights_and_padded_ld():
    q, wt, k = _int_inputs(5, 700, 64, 128)
    w_shared = np.broadcast_to(wt[0], wt.shape)
    pos = np.arange(700, dtype=np.int32)
    scores = torch.full((700, 768), np.nan, dtype=torch.float32, device="cuda:0")
    w_dev = dev(wt[0:1]).expand(700, 64)
    sma.index_scores(dev(q), w_dev, dev(k), dev(pos), scores=scores)
    got = host(scores)
    ref = _oracle(q, np.ascontiguousarray(w_shared), k, pos)
    for i in range(0, 700, 13):
        assert np.array_equal(got[i, : i + 1].astype(np.float64), ref[i])
        assert np.all(np.isnan(got[i, i + 1:]))


def test_fp8_keys_decode_shape():
    """FP8 keys + per-token scale, 64 queries at scattered positions (the
    key range is split across workgroups)."""
    w = synth.workload(5)
    n_k = 40000
    k = synth.rows(w, "k_idx", 0, n_k)
    rng = np.random.default_rng(1)
    pos = np.sort(rng.integers(0, n_k, size=64)).astype(np.int32)
    pos[-1] = n_k - 1
    q = synth.rows(synth.workload(2), "q_idx", 0, 64)
    wt = synth.rows(synth.workload(2), "w", 0, 64)
    got = _run(q, wt, k, pos)
    ref = _oracle(q, wt, k, pos, fp8=True)
    for i, p in enumerate(pos):
        r = ref[i]
        assert np.abs(got[i, : p + 1] - r).max() <= 1e-5 * np.abs(r).max(), i


def test_positions_clamped_and_empty():
    q, wt, k = _int_inputs(9, 64, 64, 128)
    pos = np.array([-5, -1, 0, 63, 64, 10 ** 6] + list(range(58)), dtype=np.int32)
    got = _run(q, wt, k, pos)
    assert np.all(np.isnan(got[0])) and np.all(np.isnan(got[1]))
    ref = _oracle(q, wt, k, np.minimum(np.maximum(pos, -1), 63))
    for i in (2, 3, 4, 5, 20):
        p = min(max(pos[i], -1), 63)
        assert np.array_equal(got[i, : p + 1].astype(np.float64), ref[i])


def test_fp8_keys_prefill_shape_exact():
    """64 heads x 128 over FP8 keys at a causal prefill shape (1,100 queries:
    many query blocks, a ragged last tile): integer q_I, keys whose codes are
    small integers with power-of-two scales, w = k/16 -> every score is exact
    in fp32, so the GPU must reproduce the oracle bit for bit."""
    rng = np.random.default_rng(77)
    n = 1100
    q = synth.to_bf16_bits(rng.integers(-3, 4, size=(n, 64, 128)).astype(np.float32))
    table = oracle.e4m3fn_table()
    ints = {int(v): c for c, v in enumerate(table[:0x7F]) if v == int(v) and v <= 4}
    ints.update({-v: c | 0x80 for v, c in list(ints.items()) if v > 0})
    keys = np.array(sorted(ints))
    lut = np.array([ints[k] for k in keys], np.uint8)
    k8 = lut[rng.integers(0, keys.size, (n, 128))]
    ks = rng.choice(np.array([0.5, 1.0, 2.0], np.float32), n)
    wt = (rng.integers(0, 17, size=(n, 64)) / 16).astype(np.float32)
    pos = np.arange(n, dtype=np.int32)
    got = _run(q, wt, (k8, ks), pos)
    ref = _oracle(q, wt, (k8, ks), pos, fp8=True)
    for i in range(n):
        assert np.array_equal(got[i, : i + 1].astype(np.float64), ref[i]), i
        assert np.all(np.isnan(got[i, i + 1:])), i
