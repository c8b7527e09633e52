"""Pins for the oracle's top-k selection (no GPU).

Reference: a full lexicographic sort (score descending, position ascending)
with numpy's lexsort, which is the definition of "the k highest, ties to the
lowest positions" written as a library call; plus invariants.
"""
import numpy as np
import pytest

import oracle
from sparse_mla_attention_index_amd import synth


def _by_full_sort(row, k):
    """Sort key: numbers before NaNs, then score descending, then position."""
    n = row.size
    m = min(k, n)
    r = row.astype(np.float64)
    isnan = np.isnan(r)
    order = np.lexsort((np.arange(n), -np.where(isnan, 0.0, r), isnan))
    out = np.full(k, -1, dtype=np.int32)
    out[:m] = np.sort(order[:m])
    return out


@pytest.mark.parametrize("kind", ["normal", "ints", "ties", "signed_zero", "nan", "nan_heavy"])
def test_matches_full_sort(kind):
    sc = synth.random_scores(11, 40, 97, kind)
    for k in (1, 5, 16, 96, 97, 200):
        for r in range(sc.shape[0]):
            n = 1 + (r * 7) % 97
            row = sc[r, :n]
            assert np.array_equal(oracle.topk_row(row, k), _by_full_sort(row, k)), (kind, k, r)


def test_invariants():
    sc = synth.random_scores(5, 64, 300, "ints")
    k = 32
    for r in range(64):
        n = 1 + (r * 37) % 300
        row = sc[r, :n]
        sel = oracle.topk_row(row, k)
        m = min(k, n)
        assert sel.shape == (k,)
        assert np.all(sel[m:] == -1)
        v = sel[:m]
        assert np.all(np.diff(v) > 0) and v.min() >= 0 and v.max() < n
        chosen = np.zeros(n, bool)
        chosen[v] = True
        if m < n:
            # every member >= every non-member; equal values: members come first
            assert row[chosen].min() >= row[~chosen].max()
            t = row[chosen].min()
            tie_pos = np.flatnonzero(row == t)
            kept = tie_pos[chosen[tie_pos]]
            assert np.array_equal(kept, tie_pos[: kept.size])


def test_signed_zero_is_one_key():
    row = np.array([-0.0, 0.0, -0.0, 0.0], dtype=np.float32)
    assert oracle.topk_row(row, 2).tolist() == [0, 1]
    row = np.array([0.0, -0.0, 1.0, -0.0], dtype=np.float32)
    assert oracle.topk_row(row, 2).tolist() == [0, 2]


def test_short_rows_take_everything():
    """A query at position p < k keeps all p+1 causal tokens (tiny workload:
    positions below 128 attend to all p+1 tokens)."""
    for p in range(0, 130):
        sel = oracle.topk_row(np.random.default_rng(p).random(p + 1), 128)
        m = min(128, p + 1)
        if p < 128:
            assert sel[:m].tolist() == list(range(p + 1))
        assert np.all(sel[:m] >= 0) and np.all(sel[m:] == -1)


def test_threshold_value():
    row = np.array([3.0, 9.0, 1.0, 9.0, 5.0])
    assert oracle.topk_threshold(row, 2) == 9.0
    assert oracle.topk_threshold(row, 3) == 5.0
    assert oracle.topk_threshold(row, 10) == 1.0


def test_nan_ranks_below_every_number():
    nan = np.float32(np.nan)
    row = np.array([nan, -np.inf, nan, 2.0, nan], dtype=np.float32)
    assert oracle.topk_row(row, 2).tolist() == [1, 3]          # -inf beats NaN
    assert oracle.topk_row(row, 3).tolist() == [0, 1, 3]       # then the lowest NaN position
    assert oracle.topk_row(row, 5).tolist() == [0, 1, 2, 3, 4]
    neg = np.array([0xFFC00000, 0x7FC00000], dtype=np.uint32).view(np.float32)   # NaNs of both signs
    assert oracle.topk_row(np.array([neg[0], neg[1], -1.0], dtype=np.float32), 2).tolist() == [0, 2]
