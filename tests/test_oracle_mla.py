"""Pins for the oracle's sparse MLA (no GPU).

* When every causal token is selected, sparse MLA is dense causal MQA
  attention (GLM-5.3 part 2, "Essayez-le": prompts within top-k may take the
  dense path unless the MQA mode is forced): compared with torch's
  scaled_dot_product_attention on the CPU.
* Absorbed form == non-absorbed form: with the latent expanded through a
  random kv_b_proj split into W_UK / W_UV (DeepSeek multi-node deployment
  page, "Parallélisme de tenseurs", "Couche MLA", "Travaux futurs"), MHA over
  k = [W_UK c, k_rope], v = W_UV c equals W_UV applied to the absorbed output.
  The absorption and output projections are the oracle's absorb_q and
  project_out, also checked by integer brute force.
* Invariants: constant values give that constant; the index order does not
  matter; one selected row returns that row's value; empty sets give 0/-inf.
"""
import numpy as np
import torch

import oracle

TAU = 1.0 / np.sqrt(192.0)


def _dense_causal_sdpa(q, kv, tau):
    """q [L, H, 576], kv [L, 576] -> [L, H, 512] via torch SDPA (float64)."""
    L, H, _ = q.shape
    qt = torch.from_numpy(q).permute(1, 0, 2).contiguous()            # [H, L, 576]
    k = torch.from_numpy(kv).unsqueeze(0).expand(H, L, 576).contiguous()
    v = torch.from_numpy(kv[:, :512]).unsqueeze(0).expand(H, L, 512).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, k, v, is_causal=True, scale=tau)
    return o.permute(1, 0, 2).numpy()


def test_dense_special_case():
    rng = np.random.default_rng(0)
    L, H = 40, 64
    q = rng.standard_normal((L, H, 576)) * 0.5
    kv = rng.standard_normal((L, 576)) * 0.5
    pos = np.arange(L)
    idx = np.full((L, 64), -1, dtype=np.int32)
    for i in range(L):
        idx[i, : i + 1] = np.arange(i + 1)
    out, lse = oracle.sparse_mla(q, kv, idx, TAU)
    ref = _dense_causal_sdpa(q, kv, TAU)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    # lse against the definition via torch.logsumexp
    z = torch.einsum("lhd,sd->lhs", torch.from_numpy(q), torch.from_numpy(kv)) * TAU
    mask = torch.arange(L)[None, :] <= torch.from_numpy(pos)[:, None]
    z = z.masked_fill(~mask[:, None, :], float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(z, dim=-1).numpy(), rtol=1e-12)


def test_absorbed_equals_expanded():
    rng = np.random.default_rng(1)
    n_k, n_q, H = 30, 5, 64
    d_nope, d_rope, d_v, d_lat = 128, 64, 128, 512
    c = rng.standard_normal((n_k, d_lat)) * 0.3           # latent from kv_a_proj
    k_rope = rng.standard_normal((n_k, d_rope)) * 0.3
    W_UK = rng.standard_normal((H, d_nope, d_lat)) * 0.05  # kv_b_proj, key half
    W_UV = rng.standard_normal((H, d_v, d_lat)) * 0.05     # kv_b_proj, value half
    q_nope = rng.standard_normal((n_q, H, d_nope))
    q_rope = rng.standard_normal((n_q, H, d_rope))
    idx = np.full((n_q, 16), -1, dtype=np.int32)
    for i in range(n_q):
        idx[i, :12] = np.sort(rng.choice(n_k, 12, replace=False))
    # absorbed: q_abs = [W_UK^T q_nope, q_rope], kv = [c, k_rope]
    q_abs = np.concatenate([oracle.absorb_q(q_nope, W_UK), q_rope], axis=-1)
    kv = np.concatenate([c, k_rope], axis=-1)
    o_lat, _ = oracle.sparse_mla(q_abs, kv, idx, TAU)
    o_abs = oracle.project_out(o_lat, W_UV)
    # expanded MHA with a mask of the selected set, via torch SDPA
    k_full = np.concatenate([np.einsum("hnl,sl->hsn", W_UK, c),
                             np.broadcast_to(k_rope, (H, n_k, d_rope))], axis=-1)   # [H, n_k, 192]
    v_full = np.einsum("hvl,sl->hsv", W_UV, c)                                       # [H, n_k, 128]
    qf = np.concatenate([q_nope, q_rope], axis=-1).transpose(1, 0, 2)                 # [H, n_q, 192]
    mask = np.zeros((n_q, n_k), dtype=bool)
    for i in range(n_q):
        mask[i, idx[i][idx[i] >= 0]] = True
    o_mha = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(np.ascontiguousarray(qf)), torch.from_numpy(np.ascontiguousarray(k_full)),
        torch.from_numpy(np.ascontiguousarray(v_full)), attn_mask=torch.from_numpy(mask), scale=TAU)
    np.testing.assert_allclose(o_abs, o_mha.permute(1, 0, 2).numpy(), rtol=1e-9, atol=1e-12)


def test_constant_value_and_order_invariance():
    rng = np.random.default_rng(2)
    n_k = 50
    q = rng.standard_normal((3, 64, 576))
    kv = rng.standard_normal((n_k, 576))
    kv[:, :512] = np.linspace(-1, 1, 512)[None, :]          # every row has the same value part
    idx = np.stack([rng.choice(n_k, 20, replace=False) for _ in range(3)]).astype(np.int32)
    out, _ = oracle.sparse_mla(q, kv, idx, TAU)
    np.testing.assert_allclose(out, np.broadcast_to(np.linspace(-1, 1, 512), out.shape), atol=1e-12)
    kv2 = rng.standard_normal((n_k, 576))
    a, la = oracle.sparse_mla(q, kv2, idx, TAU)
    b, lb = oracle.sparse_mla(q, kv2, idx[:, ::-1].copy(), TAU)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(la, lb, rtol=1e-12)


def test_single_row_and_empty():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((2, 64, 576))
    kv = rng.standard_normal((10, 576))
    idx = np.array([[7, -1, -1], [-1, -1, -1]], dtype=np.int32)
    out, lse = oracle.sparse_mla(q, kv, idx, TAU)
    np.testing.assert_allclose(out[0], np.broadcast_to(kv[7, :512], (64, 512)), rtol=1e-12)
    np.testing.assert_allclose(lse[0], TAU * (q[0] @ kv[7]), rtol=1e-12)
    assert np.all(out[1] == 0) and np.all(np.isneginf(lse[1]))


def test_softmax_weights_sum_to_one():
    """Output with value rows all ones is exactly the sum of the softmax
    weights; the log-sum-exp recovers each weight."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((4, 64, 576)) * 2
    kv = rng.standard_normal((64, 576)) * 2
    kv[:, :512] = 1.0
    idx = np.stack([np.sort(rng.choice(64, 48, replace=False)) for _ in range(4)]).astype(np.int32)
    out, lse = oracle.sparse_mla(q, kv, idx, TAU)
    assert np.abs(out - 1.0).max() < 1e-6
    for i in range(4):
        z = TAU * (q[i] @ kv[idx[i]].T)
        np.testing.assert_allclose(np.exp(z - lse[i][:, None]).sum(axis=1), 1.0, atol=1e-6)


def test_absorb_and_project_integer_bruteforce():
    """Python-integer loops on small integer inputs (exact)."""
    rng = np.random.default_rng(5)
    n, H, dn, dl, dv = 3, 2, 4, 6, 5
    qn = rng.integers(-3, 4, (n, H, dn))
    wuk = rng.integers(-3, 4, (H, dn, dl))
    ol = rng.integers(-3, 4, (n, H, dl))
    wuv = rng.integers(-3, 4, (H, dv, dl))
    ql = oracle.absorb_q(qn, wuk)
    o = oracle.project_out(ol, wuv)
    for i in range(n):
        for h in range(H):
            for c in range(dl):
                assert ql[i, h, c] == sum(int(qn[i, h, d]) * int(wuk[h, d, c]) for d in range(dn))
            for v in range(dv):
                assert o[i, h, v] == sum(int(ol[i, h, c]) * int(wuv[h, v, c]) for c in range(dl))
