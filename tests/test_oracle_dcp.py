"""Pins for the oracle's DCP shard partials and log-sum-exp merge (no GPU).

GLM-5.3 part 2, "DCP : sharder aussi le cache KV": tokens are dealt
round-robin over the ranks, each rank attends over its own shard in decode,
and the partial results are merged by their log-sum-exp.

* Identity: softmax attention over a set equals the log-sum-exp merge of
  the attentions over any partition of it, so merging every rank's partial
  gives the unsharded sparse MLA (for several rank counts, with padding and
  with queries whose tokens all sit on one rank).
* Closed form: two partials with lse = log 2 and log 6 and constant values
  1 and 3 merge to 0.25*1 + 0.75*3 = 2.5 with lse = log 8.
* Special cases: one rank is the unsharded attention; an all-empty (query,
  head) stays 0 / -inf; a rank's rows are tokens rank, rank + P, ...
"""
import numpy as np
import pytest

import oracle

TAU = 1.0 / np.sqrt(192.0)


def _case(seed, n_q=5, n_k=97, H=64, K=24):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n_q, H, 576)) * 0.5
    kv = rng.standard_normal((n_k, 576)) * 0.5
    idx = np.full((n_q, K), -1, dtype=np.int64)
    for i in range(n_q):
        m = int(rng.integers(1, K + 1))
        idx[i, :m] = np.sort(rng.choice(n_k, size=m, replace=False))
    return q, kv, idx


@pytest.mark.parametrize("P", [1, 2, 3, 8])
def test_merge_of_shards_is_unsharded(P):
    q, kv, idx = _case(P)
    idx[0, :] = -1                       # an empty query
    idx[1, :3] = [P, 2 * P, 5 * P]       # every token on rank 0
    idx[1, 3:] = -1
    full_o, full_lse = oracle.sparse_mla(q, kv, idx, TAU)
    parts, lses = zip(*[oracle.dcp_shard_partial(r, P, q, kv, idx, TAU) for r in range(P)])
    o, lse = oracle.lse_merge(np.stack(parts), np.stack(lses))
    assert np.allclose(o, full_o, rtol=1e-12, atol=1e-12)
    fin = np.isfinite(full_lse)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.allclose(lse[fin], full_lse[fin], rtol=1e-12, atol=1e-12)
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))


def test_closed_form_two_partials():
    parts = np.stack([np.ones((1, 2, 4)), 3 * np.ones((1, 2, 4))])
    lses = np.log(np.array([[[2.0, 2.0]], [[6.0, 6.0]]]))
    o, lse = oracle.lse_merge(parts, lses)
    assert np.allclose(o, 2.5) and np.allclose(lse, np.log(8.0))


def test_empty_partials_and_single_rank():
    parts = np.zeros((3, 1, 1, 2))
    parts[1] = 7.0
    lses = np.full((3, 1, 1), -np.inf)
    lses[1] = 0.3
    o, lse = oracle.lse_merge(parts, lses)     # only rank 1 holds anything
    assert np.allclose(o, 7.0) and np.allclose(lse, 0.3)
    o, lse = oracle.lse_merge(np.zeros((2, 1, 1, 2)), np.full((2, 1, 1), -np.inf))
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    q, kv, idx = _case(5)
    o1, l1 = oracle.dcp_shard_partial(0, 1, q, kv, idx, TAU)
    o2, l2 = oracle.sparse_mla(q, kv, idx, TAU)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_shard_rows_round_robin():
    kv = np.arange(10 * 3, dtype=np.float64).reshape(10, 3)
    for r in range(4):
        rows = oracle.dcp_shard_rows(r, 4, kv)
        assert np.array_equal(rows, kv[[s for s in range(10) if s % 4 == r]])
    with pytest.raises(ValueError):
        oracle.dcp_shard_rows(4, 4, kv)


def test_partial_reads_the_same_rows_as_the_shard():
    """The rank's partial over global positions equals attention over its
    own shard with local rows s // P."""
    P, r = 4, 2
    q, kv, idx = _case(9)
    o, lse = oracle.dcp_shard_partial(r, P, q, kv, idx, TAU)
    local = np.where((idx >= 0) & (idx % P == r), idx // P, -1)
    o2, lse2 = oracle.sparse_mla(q, oracle.dcp_shard_rows(r, P, kv), local, TAU)
    assert np.allclose(o, o2, rtol=0, atol=0) and np.array_equal(lse, lse2)
