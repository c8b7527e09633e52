"""Pins for the oracle's dense MHA prefill (no GPU).

The path: for prompts that fit inside top-k, prefill projects the latent
into per-head keys and values first and runs dense causal multi-head
attention (GLM-5.3 part 2, "Essayez-le"; DeepSeek multi-node page,
"Travaux futurs", "Couche MLA").

* Against torch's scaled_dot_product_attention on the CPU (float64), with
  the keys and values built by torch matmuls from random W_UK / W_UV, for a
  contiguous causal prompt and for scattered query positions (an explicit
  boolean mask), including an empty prefix.
* Against the absorbed sparse path of the same attention: when every causal
  token is selected, W_UV applied to sparse MLA over the absorbed query
  [W_UK^T q_nope, q_rope] equals dense MHA, outputs and log-sum-exp (the
  identity the pages' MQA mode relies on), through the oracle's own
  absorb_q / sparse_mla / project_out, each pinned on its own.
* A dropped rope term, a wrong scale, a transposed W, or an off-by-one
  causal bound changes the result: checked on planted variants.
"""
import numpy as np
import pytest
import torch

import oracle

TAU = 1.0 / np.sqrt(192.0)


def _inputs(n_k, n_q, H=8, seed=0):
    rng = np.random.default_rng(seed)
    kv = rng.standard_normal((n_k, 576)) * 0.5
    w_uk = rng.standard_normal((H, 128, 512)) * 0.05
    w_uv = rng.standard_normal((H, 128, 512)) * 0.05
    q = rng.standard_normal((n_q, H, 192)) * 0.5
    return q, kv, w_uk, w_uv


def _sdpa(q, kv, w_uk, w_uv, q_pos):
    """Dense MHA through torch: K = [c W_UK^T, rope], V = c W_UV^T per head."""
    c = torch.from_numpy(kv[:, :512])
    rope = torch.from_numpy(kv[:, 512:])
    H = w_uk.shape[0]
    n_k = kv.shape[0]
    k = torch.cat([torch.matmul(c, torch.from_numpy(w_uk).transpose(1, 2)),          # [H, n_k, 128]
                   rope.unsqueeze(0).expand(H, n_k, 64)], dim=2).contiguous()       # [H, n_k, 192]
    v = torch.matmul(c, torch.from_numpy(w_uv).transpose(1, 2)).contiguous()        # [H, n_k, 128]
    qt = torch.from_numpy(q).permute(1, 0, 2).contiguous()                          # [H, n_q, 192]
    mask = torch.arange(n_k)[None, :] <= torch.from_numpy(np.asarray(q_pos))[:, None]   # [n_q, n_k]
    o = torch.nn.functional.scaled_dot_product_attention(qt, k, v, attn_mask=mask, scale=TAU)
    return o.permute(1, 0, 2).numpy()


def test_contiguous_prompt_matches_sdpa_causal():
    q, kv, w_uk, w_uv = _inputs(48, 48)
    pos = np.arange(48)
    out, _ = oracle.dense_mha_prefill(q, kv, w_uk, w_uv, pos, TAU)
    c = torch.from_numpy(kv[:, :512])
    H = w_uk.shape[0]
    k = torch.cat([torch.matmul(c, torch.from_numpy(w_uk).transpose(1, 2)),
                   torch.from_numpy(kv[:, 512:]).unsqueeze(0).expand(H, 48, 64)], dim=2).contiguous()
    v = torch.matmul(c, torch.from_numpy(w_uv).transpose(1, 2)).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q).permute(1, 0, 2).contiguous(), k, v,
                                                           is_causal=True, scale=TAU).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


def test_scattered_positions_match_sdpa_mask():
    q, kv, w_uk, w_uv = _inputs(60, 7, seed=3)
    pos = np.array([0, 59, 17, 31, 1, 45, 8])
    out, lse = oracle.dense_mha_prefill(q, kv, w_uk, w_uv, pos, TAU)
    np.testing.assert_allclose(out, _sdpa(q, kv, w_uk, w_uv, pos), rtol=1e-10, atol=1e-12)
    # query 0 attends to token 0 alone: its value row exactly, lse = its logit
    v0 = np.einsum("c,hdc->hd", kv[0, :512], w_uv)
    np.testing.assert_allclose(out[0], v0, rtol=1e-12, atol=1e-14)


def test_empty_prefix():
    q, kv, w_uk, w_uv = _inputs(10, 2, seed=4)
    out, lse = oracle.dense_mha_prefill(q, kv, w_uk, w_uv, np.array([-1, 3]), TAU)
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0])) and np.all(np.isfinite(lse[1]))


@pytest.mark.parametrize("H", [8, 64])
def test_equals_absorbed_sparse_path_when_all_selected(H):
    n_k = 40
    q, kv, w_uk, w_uv = _inputs(n_k, n_k, H=H, seed=5 + H)
    pos = np.arange(n_k)
    out, lse = oracle.dense_mha_prefill(q, kv, w_uk, w_uv, pos, TAU)
    q_abs = np.concatenate([oracle.absorb_q(q[:, :, :128], w_uk), q[:, :, 128:]], axis=2)   # [n, H, 576]
    idx = np.full((n_k, 64), -1, dtype=np.int32)
    for i in range(n_k):
        idx[i, : i + 1] = np.arange(i + 1)           # every causal token (top_k >= prompt)
    o_lat, lse_s = oracle.sparse_mla(q_abs, kv, idx, TAU)
    np.testing.assert_allclose(oracle.project_out(o_lat, w_uv), out, rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(lse_s, lse, rtol=1e-12, atol=1e-12)


def test_planted_mistakes_are_caught():
    """Each plausible slip, written as a variant here, moves the result away
    from the SDPA reference by far more than the pins' tolerance."""
    q, kv, w_uk, w_uv = _inputs(24, 24, seed=9)
    pos = np.arange(24)
    ref = _sdpa(q, kv, w_uk, w_uv, pos)
    variants = {
        "rope dropped": (np.concatenate([q[:, :, :128], 0 * q[:, :, 128:]], axis=2), kv, w_uk, w_uv, pos, TAU),
        "scale 1/sqrt(128)": (q, kv, w_uk, w_uv, pos, 1 / np.sqrt(128.0)),
        "W_UK and W_UV swapped": (q, kv, w_uv, w_uk, pos, TAU),
        "causal bound off by one": (q, kv, w_uk, w_uv, np.maximum(pos - 1, 0), TAU),
    }
    for name, args in variants.items():
        got, _ = oracle.dense_mha_prefill(*args)
        assert np.abs(got - ref).max() > 1e-6, name
