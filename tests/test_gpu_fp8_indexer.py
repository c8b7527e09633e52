"""GPU parity of the FP8 indexer: sma_quantize_fp8_rows (bit-exact codes and
scales against the oracle's quantiser), sma_index_scores_fp8 (exact on
integer-valued codes, within fp32 accumulation error on N(0,1) data, at the
16K prompt's full size on sampled rows) and sma_prefill_fp8_indexer."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_index_amd as sma
from sparse_mla_attention_index_amd import synth
from _gpuhelp import check_topk_threshold_rule, dev, host, out_f64

pytestmark = pytest.mark.gpu


def _bf16_rows(x):
    """fp32 values -> (bf16 bit patterns, the fp32 values they hold)."""
    bits = synth.to_bf16_bits(np.asarray(x, dtype=np.float32))
    return bits, oracle.bf16_bits_to_f64(bits).astype(np.float32)


def _quant_gpu(bits):
    codes, scale = sma.quantize_fp8_rows(dev(bits))
    torch.cuda.synchronize()
    return host(codes), host(scale)


@pytest.mark.parametrize("d", [128, 64])
def test_quantize_rows_bitexact(d):
    rng = np.random.default_rng(d)
    n = 2000 + 37   # several workgroups and a ragged tail
    x = rng.standard_normal((n, d)).astype(np.float32) * np.exp2(rng.integers(-30, 30, (n, 1)))
    x[3] = 0.0                          # zero row: scale 0, codes 0
    x[4, :] = -1e-3
    x[4, 7] = -5.0                      # amax element negative
    x[5, ::3] = 0.0                     # zeros among values
    bits, vals = _bf16_rows(x)
    codes, scale = _quant_gpu(bits)
    ref_c, ref_s = oracle.quantize_fp8_rows(vals)
    assert np.array_equal(scale, ref_s)
    assert np.array_equal(codes, ref_c)


def test_quantize_rows_ties_and_subnormals():
    """Rows whose amax is 448 have scale 1, so the row's values reach the
    convert unchanged: every midpoint between neighbouring e4m3 codes (a tie,
    to the even code) and the subnormal range, both signs."""
    pos = np.sort(oracle.e4m3fn_table()[:0x7F])           # 0 .. 448
    mid = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)   # 5 significant bits: exact in bf16
    vals = np.concatenate([mid, -mid, pos[1:16].astype(np.float32) * 0.75])
    n_rows = -(-vals.size // 127)
    x = np.zeros((n_rows, 128), np.float32)
    x[:, 0] = 448.0
    flat = np.zeros(n_rows * 127, np.float32)
    flat[: vals.size] = vals
    x[:, 1:] = flat.reshape(n_rows, 127)
    bits, v = _bf16_rows(x)
    assert np.array_equal(v, x)
    codes, scale = _quant_gpu(bits)
    ref_c, ref_s = oracle.quantize_fp8_rows(v)
    assert np.all(scale == 1.0) and np.array_equal(scale, ref_s)
    assert np.array_equal(codes, ref_c)


def _int_fp8_inputs(seed, n_q, n_k):
    """Codes of small integers, power-of-two scales, w = k/16: every score
    is an exact fp32 number."""
    rng = np.random.default_rng(seed)
    table = oracle.e4m3fn_table()
    ints = {int(v): c for c, v in enumerate(table[:0x7F]) if v == int(v) and v <= 4}
    ints.update({-v: c | 0x80 for v, c in list(ints.items()) if v > 0})
    keys = np.array(sorted(ints))
    lut = np.array([ints[k] for k in keys], np.uint8)
    q8 = lut[rng.integers(0, keys.size, (n_q, 64, 128))]
    k8 = lut[rng.integers(0, keys.size, (n_k, 128))]
    qs = rng.choice(np.array([0.5, 1.0, 2.0], np.float32), (n_q, 64))
    ks = rng.choice(np.array([0.5, 1.0], np.float32), n_k)
    w = (rng.integers(0, 17, (n_q, 64)) / 16).astype(np.float32)
    return q8, qs, w, k8, ks


def _scores_gpu(q8, qs, w, k8, ks, pos, ld=None):
    n_q, n_k = q8.shape[0], k8.shape[0]
    scores = torch.full((n_q, ld or n_k), np.nan, dtype=torch.float32, device="cuda:0")
    sma.index_scores_fp8(dev(q8), dev(qs), dev(w), dev(k8), dev(ks), dev(pos), scores=scores)
    torch.cuda.synchronize()
    return host(scores)


def test_fp8_scores_integer_exact():
    n = 1037    # several 128-key tiles, 8-query blocks and a ragged tail
    q8, qs, w, k8, ks = _int_fp8_inputs(1, n, n)
    pos = np.arange(n, dtype=np.int32)
    got = _scores_gpu(q8, qs, w, k8, ks, pos, ld=n + 5)
    ref = oracle.index_scores_fp8(q8, qs, w, k8, ks, pos)
    for i in range(n):
        assert np.array_equal(got[i, : i + 1].astype(np.float64), ref[i]), i
        assert np.all(np.isnan(got[i, i + 1:])), i


def test_fp8_scores_normal_tolerance():
    """16K-workload distributions, quantised by the input generator; fp32
    accumulation against the float64 oracle on the same codes."""
    w = synth.workload(2)
    n = 2500
    q8, qs = synth.to_fp8_rows(oracle.bf16_bits_to_f64(synth.rows(w, "q_idx", 0, n).reshape(-1, 128)))
    q8, qs = q8.reshape(n, 64, 128), qs.reshape(n, 64)
    wt = synth.rows(w, "w", 0, n)
    kb = oracle.bf16_bits_to_f64(synth.rows(w, "k_idx", 0, n)).astype(np.float32)
    k8, ks = synth.to_fp8_rows(kb)
    pos = np.arange(n, dtype=np.int32)
    got = _scores_gpu(q8, qs, wt, k8, ks, pos)
    rows = list(range(0, n, 11)) + [n - 1]
    _check_fp32_bound(got, rows, q8, qs, wt, k8, ks, pos)


U32 = 2.0 ** -24


def _check_fp32_bound(got, rows, q8, qs, w, k8, ks, pos):
    """Element-wise bound of fp32 evaluation in any order: a 128-term dot
    product, a weight times a scale, a 64-term head sum and the key scale
    give |error| <= (127 + 63 + 3) u B with B = sum_h |w_h| sq_h sk sum_d
    |q_d k_d| (the oracle's scores of the magnitudes), u = 2^-24."""
    ref = oracle.index_scores_fp8(q8[rows], qs[rows], w[rows], k8, ks, pos[rows])
    mag = oracle.index_scores_fp8(q8[rows] & 0x7F, qs[rows], np.abs(w[rows]), k8 & 0x7F, ks, pos[rows])
    worst = 0.0
    for i, r, b in zip(rows, ref, mag):
        err = np.abs(got[i, : pos[i] + 1] - r)
        worst = max(worst, float(np.max(err / (U32 * b + 1e-300))))
    assert worst <= 193, f"error reaches {worst:.1f} u B (bound 193)"
    return worst


def test_fp8_scores_decode_shape_and_clamps():
    """64 queries at scattered positions over 40,000 keys (the key range is
    split across workgroups), plus clamped and empty positions."""
    rng = np.random.default_rng(3)
    n_k = 40000
    q8, qs, w, k8, ks = _int_fp8_inputs(4, 64, n_k)
    pos = np.sort(rng.integers(0, n_k, size=64)).astype(np.int32)
    pos[:3] = [-7, -1, 0]
    pos[-2:] = [n_k - 1, 10 ** 9]
    got = _scores_gpu(q8, qs, w, k8, ks, pos)
    assert np.all(np.isnan(got[0])) and np.all(np.isnan(got[1]))
    cp = np.clip(pos, -1, n_k - 1)
    ref = oracle.index_scores_fp8(q8[2:], qs[2:], w[2:], k8, ks, cp[2:])
    for i, r in zip(range(2, 64), ref):
        assert np.array_equal(got[i, : cp[i] + 1].astype(np.float64), r), i
        assert np.all(np.isnan(got[i, cp[i] + 1:])), i


def test_gpu_quantiser_feeds_fp8_indexer():
    """bf16 q_I / k_I -> GPU quantiser -> GPU FP8 scores equals the oracle's
    quantiser -> oracle FP8 scores (the codes agree bit for bit)."""
    w = synth.workload(2)
    n = 700
    qb = synth.rows(w, "q_idx", 0, n)
    kb = synth.rows(w, "k_idx", 0, n)
    wt = synth.rows(w, "w", 0, n)
    q8d, qsd = sma.quantize_fp8_rows(dev(qb))
    k8d, ksd = sma.quantize_fp8_rows(dev(kb))
    pos = np.arange(n, dtype=np.int32)
    scores = torch.full((n, n), np.nan, dtype=torch.float32, device="cuda:0")
    sma.index_scores_fp8(q8d, qsd, dev(wt), k8d, ksd, dev(pos), scores=scores)
    got = host(scores)
    q8, qs = oracle.quantize_fp8_rows(oracle.bf16_bits_to_f64(qb.reshape(-1, 128)))
    k8, ks = oracle.quantize_fp8_rows(oracle.bf16_bits_to_f64(kb))
    assert np.array_equal(host(q8d).reshape(-1, 128), q8) and np.array_equal(host(qsd).reshape(-1), qs)
    assert np.array_equal(host(k8d), k8) and np.array_equal(host(ksd), ks)
    rows = list(range(0, n, 13)) + [n - 1]
    ref = oracle.index_scores_fp8(q8.reshape(n, 64, 128)[rows], qs.reshape(n, 64)[rows], wt[rows], k8, ks,
                                  pos[rows])
    _check_fp32_bound(got, rows, q8.reshape(n, 64, 128), qs.reshape(n, 64), wt, k8, ks, pos)


def test_fp8_scores_full_16k_sampled():
    """The 16K prompt at full size (all 16,384 query rows in one launch),
    checked on sampled rows against the oracle."""
    w = synth.workload(2)
    n = w.n_keys
    qb = synth.rows(w, "q_idx", 0, n)
    kb = synth.rows(w, "k_idx", 0, n)
    wt = synth.rows(w, "w", 0, n)
    q8d, qsd = sma.quantize_fp8_rows(dev(qb))
    k8d, ksd = sma.quantize_fp8_rows(dev(kb))
    pos = np.arange(n, dtype=np.int32)
    got = sma.index_scores_fp8(q8d, qsd, dev(wt), k8d, ksd, dev(pos))
    rows = np.array([0, 1, 777, 4095, 8191, 12000, n - 2, n - 1])
    g = host(got[torch.from_numpy(rows).to("cuda:0")])
    k8, ks = oracle.quantize_fp8_rows(oracle.bf16_bits_to_f64(kb))
    q8, qs = oracle.quantize_fp8_rows(oracle.bf16_bits_to_f64(qb[rows].reshape(-1, 128)))
    gfull = np.full((rows.size, n), np.nan, np.float32)
    gfull[:] = g
    _check_fp32_bound(gfull, list(range(rows.size)), q8.reshape(rows.size, 64, 128), qs.reshape(rows.size, 64),
                      wt[rows], k8, ks, pos[rows])


def _fp8_prefill_inputs(w, n, seed_int=None):
    pos = np.arange(n, dtype=np.int32)
    q = synth.rows(w, "q", 0, n)
    kv = synth.rows(w, "kv", 0, n)
    if seed_int is not None:
        q8, qs, wt, k8, ks = _int_fp8_inputs(seed_int, n, n)
    else:
        q8, qs = synth.to_fp8_rows(oracle.bf16_bits_to_f64(synth.rows(w, "q_idx", 0, n).reshape(-1, 128)))
        q8, qs = q8.reshape(n, 64, 128), qs.reshape(n, 64)
        k8, ks = synth.to_fp8_rows(oracle.bf16_bits_to_f64(synth.rows(w, "k_idx", 0, n)))
        wt = synth.rows(w, "w", 0, n)
    return dict(pos=pos, q=q, kv=kv, q8=q8, qs=qs, w=wt, k8=k8, ks=ks)


def _fp8_prefill_gpu(w, d, top_k, workspace=None):
    n = d["pos"].size
    idx = torch.empty((n, top_k), dtype=torch.int32, device="cuda:0")
    out, lse, _ = sma.prefill_fp8_indexer(dev(d["q8"]), dev(d["qs"]), dev(d["w"]), dev(d["k8"]), dev(d["ks"]),
                                          dev(d["q"]), dev(d["kv"]), dev(d["pos"]), top_k, w.sm_scale,
                                          want_lse=True, idx_out=idx, workspace=workspace)
    torch.cuda.synchronize()
    return out, lse, idx


def test_fp8_prefill_integer_exact_lists():
    """Exact FP8 indexer scores -> the index lists equal the oracle's; the
    attention output is within 1e-2 of max|ref| (bf16 output)."""
    w = synth.workload(2)
    n, top_k = 1100, 256
    d = _fp8_prefill_inputs(w, n, seed_int=6)
    out, lse, idx = _fp8_prefill_gpu(w, d, top_k)
    sc = oracle.index_scores_fp8(d["q8"], d["qs"], d["w"], d["k8"], d["ks"], d["pos"])
    ref_idx = oracle.topk_select(sc, top_k)
    assert np.array_equal(host(idx), ref_idx)
    rows = list(range(0, n, 37)) + [n - 1]
    f = oracle.bf16_bits_to_f64
    ref_out, ref_lse = oracle.sparse_mla(f(d["q"][rows]), f(d["kv"]), ref_idx[rows], w.sm_scale)
    got = out_f64(out)[rows]
    assert np.abs(got - ref_out).max() <= 1e-2 * np.abs(ref_out).max()
    assert np.abs(host(lse)[rows] - ref_lse).max() < 2e-3


def test_fp8_prefill_normal_threshold_rule_and_components():
    """N(0,1) data: the selections follow the 1e-3 threshold rule against
    the oracle's FP8 scores, and the composed call equals the three calls
    made one by one, bit for bit, whatever the workspace."""
    w = synth.workload(2)
    n = 3000
    d = _fp8_prefill_inputs(w, n)
    out, lse, idx = _fp8_prefill_gpu(w, d, w.top_k)
    gi = host(idx)
    rows = list(range(0, n, 41)) + [n - 1]
    sc = oracle.index_scores_fp8(d["q8"][rows], d["qs"][rows], d["w"][rows], d["k8"], d["ks"], d["pos"][rows])
    for r, s in zip(rows, sc):
        check_topk_threshold_rule(gi[r], s, w.top_k)
    scores = sma.index_scores_fp8(dev(d["q8"]), dev(d["qs"]), dev(d["w"]), dev(d["k8"]), dev(d["ks"]),
                                  dev(d["pos"]))
    idx2 = sma.topk_select(scores, dev(d["pos"]), w.top_k)
    out2, lse2 = sma.sparse_mla_prefill(dev(d["q"]), dev(d["kv"]), idx2, w.sm_scale, want_lse=True)
    assert torch.equal(idx, idx2) and torch.equal(out, out2) and torch.equal(lse, lse2)
    ws = torch.empty(sma.workspace_bytes(3, n, n, w.top_k), dtype=torch.uint8, device="cuda:0")
    out3, lse3, idx3 = _fp8_prefill_gpu(w, d, w.top_k, workspace=ws)
    assert torch.equal(idx, idx3) and torch.equal(out, out3) and torch.equal(lse, lse3)
