"""Pins for the oracle's indexer scores (no GPU).

What fixes the values: on integer-valued q_I/k_I and w = k/16 (the tiny
workload's recipe) every score is an exact multiple of 1/16 well below 2^24,
so Python integer arithmetic gives the exact result to compare against.
"""
import numpy as np

import oracle
from sparse_mla_attention_index_amd import synth


def _exact_scores_int(q_int, w16_int, k_int, p):
    """Brute force in Python ints: 16 * I[s] for s = 0..p (w = w16/16)."""
    H, D = len(q_int), len(q_int[0])
    res = []
    for s in range(p + 1):
        tot = 0
        for h in range(H):
            d = 0
            for j in range(D):
                d += q_int[h][j] * k_int[s][j]
            if d > 0:
                tot += w16_int[h] * d
        res.append(tot)
    return res


def test_tiny_integer_bruteforce():
    rng = np.random.default_rng(7)
    n_q, n_k, H, D = 6, 24, 3, 5
    q = rng.integers(-3, 4, size=(n_q, H, D))
    k = rng.integers(-3, 4, size=(n_k, D))
    w16 = rng.integers(0, 17, size=(n_q, H))
    pos = np.array([0, 1, 5, 11, 17, 23])
    got = oracle.index_scores(q.astype(np.float64), w16 / 16.0, k.astype(np.float64), pos)
    for i in range(n_q):
        exact = _exact_scores_int(q[i].tolist(), w16[i].tolist(), k.tolist(), int(pos[i]))
        assert got[i].shape == (pos[i] + 1,)
        assert [int(round(v * 16)) for v in got[i]] == exact
        assert np.array_equal(got[i] * 16, np.array(exact, dtype=np.float64))


def test_tiny_workload_rows_exact():
    """Sampled queries of the tiny workload (8 heads x 64, integer inputs)."""
    w = synth.workload(1)
    k = oracle.bf16_bits_to_f64(synth.rows(w, "k_idx", 0, w.n_keys))
    for p in (0, 127, 300, 511):
        q = oracle.bf16_bits_to_f64(synth.rows(w, "q_idx", p, p + 1))
        wt = synth.rows(w, "w", p, p + 1).astype(np.float64)
        assert np.all(wt * 16 == np.round(wt * 16))
        got = oracle.index_scores(q, wt, k, np.array([p]))[0]
        exact = _exact_scores_int(q[0].astype(int).tolist(), (wt[0] * 16).astype(int).tolist(),
                                  k[: p + 1].astype(int).tolist(), p)
        assert np.array_equal(got * 16, np.array(exact, dtype=np.float64))


def test_relu_and_head_weight():
    """One head with a negative dot contributes nothing; w weights heads."""
    q = np.array([[[1.0, 0.0], [-1.0, 0.0]]])     # 2 heads
    k = np.array([[2.0, 5.0], [-3.0, 1.0]])
    w = np.array([[0.5, 4.0]])
    s = oracle.index_scores(q, w, k, np.array([1]))[0]
    # key 0: head0 dot=2 -> 0.5*2; head1 dot=-2 -> 0. key 1: head0 -3 -> 0; head1 3 -> 4*3
    assert s.tolist() == [1.0, 12.0]


def test_causal_length_includes_self():
    q = np.ones((3, 1, 2))
    k = np.ones((10, 2))
    w = np.ones((3, 1))
    pos = np.array([0, 4, 9])
    out = oracle.index_scores(q, w, k, pos)
    assert [o.size for o in out] == [1, 5, 10]


def test_positive_scale_homogeneity():
    """Scaling keys by s > 0 scales every score by s (what lets a per-token
    FP8 scale be applied after the head reduce)."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal((4, 8, 16))
    k = rng.standard_normal((32, 16))
    w = rng.random((4, 8))
    pos = np.array([3, 10, 20, 31])
    sc = rng.random(32) * 3 + 0.1
    a = oracle.index_scores(q, w, k * sc[:, None], pos)
    b = oracle.index_scores(q, w, k, pos)
    for x, y, p in zip(a, b, pos):
        np.testing.assert_allclose(x, y * sc[: p + 1], rtol=1e-12)


def test_distinguishes_heads_from_dims():
    """A score must pair head h of the query with the key's dims: with one
    nonzero head the score is that head's ReLU dot alone."""
    q = np.zeros((1, 4, 3))
    q[0, 2] = [1.0, 2.0, 3.0]
    k = np.array([[1.0, 1.0, 1.0], [0.0, 0.0, -1.0]])
    w = np.array([[1.0, 1.0, 2.0, 1.0]])
    s = oracle.index_scores(q, w, k, np.array([1]))[0]
    assert s.tolist() == [12.0, 0.0]
