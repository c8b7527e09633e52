"""GPU parity of the absorption products (sma_absorb_q, sma_project_out)
against the oracle: exact on small-integer inputs, element-wise within the
fp32-accumulation-plus-bf16-rounding bound on N(0,1) data, writing in place
into a sparse-MLA query, and the absorbed attention end to end."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_index_amd as sma
from sparse_mla_attention_index_amd import synth
from _gpuhelp import bf16_out_to_f64, dev, host

pytestmark = pytest.mark.gpu
TAU = 1.0 / np.sqrt(192.0)
U32 = 2.0 ** -24


def _bf16(x):
    return synth.to_bf16_bits(np.asarray(x, np.float32))


def _vals(bits):
    return oracle.bf16_bits_to_f64(bits)


def test_absorb_q_integer_exact_in_place():
    """Entries in {-1, 0, 1}: every sum (|.| <= 128) is exact in fp32 and in
    bf16.  Written into a [n, 64, 576] query: dims 512..575 untouched."""
    rng = np.random.default_rng(1)
    n, H = 300, 64                      # two full 128-row tiles and a ragged one
    qn = _bf16(rng.integers(-1, 2, (n, H, 128)))
    wuk = _bf16(rng.integers(-1, 2, (H, 128, 512)))
    q = torch.full((n, H, 576), 7.0, dtype=torch.bfloat16, device="cuda:0")
    sma.absorb_q(dev(qn), dev(wuk), out=q)
    got = bf16_out_to_f64(q)
    ref = oracle.absorb_q(_vals(qn), _vals(wuk))
    assert np.array_equal(got[:, :, :512], ref)
    assert np.all(got[:, :, 512:] == 7.0)


def test_project_out_integer_exact():
    rng = np.random.default_rng(2)
    n, H = 200, 64
    ol = _bf16(rng.integers(-1, 2, (n, H, 512)))
    w = rng.integers(-1, 2, (H, 128, 512)) * (rng.random((H, 128, 512)) < 0.25)
    wuv = _bf16(w)
    ref = oracle.project_out(_vals(ol), _vals(wuv))
    assert np.abs(ref).max() <= 256      # exact in bf16
    got = bf16_out_to_f64(sma.project_out(dev(ol), dev(wuv)))
    assert np.array_equal(got, ref)


def _bound_check(got, ref, mag, k):
    """|got - ref| <= (k - 1) u B + (half a bf16 ulp of the fp32 result):
    B = the products' magnitudes summed, u = 2^-24."""
    err = np.abs(got - ref)
    lim = (k - 1) * U32 * mag + 2.0 ** -8 * (np.abs(ref) + (k - 1) * U32 * mag)
    worst = float(np.max(err / (lim + 1e-300)))
    assert worst <= 1.0, worst


@pytest.mark.parametrize("heads", [64, 16])
def test_absorb_and_project_normal(heads):
    rng = np.random.default_rng(3 + heads)
    n = 777
    qn = _bf16(rng.standard_normal((n, heads, 128)))
    wuk = _bf16(rng.standard_normal((heads, 128, 512)) * 0.05)
    ol = _bf16(rng.standard_normal((n, heads, 512)) * 0.1)
    wuv = _bf16(rng.standard_normal((heads, 128, 512)) * 0.05)
    got_q = bf16_out_to_f64(sma.absorb_q(dev(qn), dev(wuk)))
    _bound_check(got_q, oracle.absorb_q(_vals(qn), _vals(wuk)),
                 oracle.absorb_q(np.abs(_vals(qn)), np.abs(_vals(wuk))), 128)
    got_o = bf16_out_to_f64(sma.project_out(dev(ol), dev(wuv)))
    _bound_check(got_o, oracle.project_out(_vals(ol), _vals(wuv)),
                 oracle.project_out(np.abs(_vals(ol)), np.abs(_vals(wuv))), 512)


def test_absorbed_attention_end_to_end():
    """q_nope, q_rope and the latent rows -> absorb_q into the query ->
    sparse MLA -> project_out, against the oracle's same three steps."""
    rng = np.random.default_rng(4)
    n, n_k, H, top_k = 150, 2000, 64, 256
    qn = _bf16(rng.standard_normal((n, H, 128)))
    qr = _bf16(rng.standard_normal((n, H, 64)) * 0.5)
    wuk = _bf16(rng.standard_normal((H, 128, 512)) * 0.05)
    wuv = _bf16(rng.standard_normal((H, 128, 512)) * 0.05)
    kv = _bf16(rng.standard_normal((n_k, 576)) * 0.3)
    idx = np.full((n, top_k), -1, np.int32)
    for i in range(n):
        m = int(rng.integers(1, top_k + 1))
        idx[i, :m] = np.sort(rng.choice(n_k, m, replace=False))
    q = torch.empty((n, H, 576), dtype=torch.bfloat16, device="cuda:0")
    q[:, :, 512:] = dev(qr).view(torch.bfloat16)
    sma.absorb_q(dev(qn), dev(wuk), out=q)
    o_lat, _ = sma.sparse_mla_prefill(q, dev(kv), dev(idx), TAU)
    o = bf16_out_to_f64(sma.project_out(o_lat, dev(wuv)))
    q_ref = np.concatenate([oracle.absorb_q(_vals(qn), _vals(wuk)), _vals(qr)], axis=-1)
    ol_ref, _ = oracle.sparse_mla(q_ref, _vals(kv), idx, TAU)
    o_ref = oracle.project_out(ol_ref, _vals(wuv))
    assert np.abs(o - o_ref).max() <= 1e-2 * np.abs(o_ref).max()
