"""GPU parity of sma_topk_select: bit-exact index lists against the oracle
on the same fp32 scores (the selection is unique given the scores)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_mla_attention_index_amd as sma
from sparse_mla_attention_index_amd import synth
from _gpuhelp import dev, host

pytestmark = pytest.mark.gpu


def _positions(n_rows, n_k, top_k, seed):
    rng = np.random.default_rng(seed)
    pos = rng.integers(0, n_k, size=n_rows)
    fixed = [0, 1, top_k - 2, top_k - 1, top_k, top_k + 1, n_k - 1, n_k // 2]
    pos[: len(fixed)] = np.clip(fixed, 0, n_k - 1)
    return pos.astype(np.int32)


@pytest.mark.parametrize("kind", ["normal", "ints", "ties", "signed_zero", "nan", "nan_heavy"])
# rows of <= 32,768 scores, <= 65,536 and longer take three different filtered kernels
@pytest.mark.parametrize("n_k,top_k", [(300, 128), (5000, 2048), (20000, 2048), (32768, 2048), (40000, 1),
                                       (50000, 2048), (70000, 2048), (140000, 2048)])
def test_topk_exact(kind, n_k, top_k):
    n_rows = 24
    sc = synth.random_scores(n_k % 1000 + len(kind), n_rows, n_k, kind)
    pos = _positions(n_rows, n_k, top_k, n_k)
    idx = sma.topk_select(dev(sc), dev(pos), top_k)
    got = host(idx)
    for r in range(n_rows):
        ref = oracle.topk_row(sc[r, : pos[r] + 1], top_k)
        assert np.array_equal(got[r], ref), (kind, n_k, top_k, r, pos[r])


@pytest.mark.parametrize("pad,kind", [(1, "normal"), (3, "normal"), (64, "normal"), (1, "nan"), (3, "nan_heavy")])
def test_topk_row_stride(pad, kind):
    """Rows with a leading dimension larger than n_k (aligned or not; an
    unaligned row takes the streaming selection)."""
    n_k, top_k, n_rows = 9000, 512, 16
    sc = synth.random_scores(77, n_rows, n_k + pad, kind)
    pos = _positions(n_rows, n_k, top_k, pad)
    t = dev(sc)
    idx = sma.topk_select(t, dev(pos), top_k, n_k=n_k)
    got = host(idx)
    for r in range(n_rows):
        assert np.array_equal(got[r], oracle.topk_row(sc[r, : pos[r] + 1], top_k)), r


def test_topk_clamped_positions():
    n_k, top_k = 3000, 100
    sc = synth.random_scores(3, 4, n_k, "ints")
    pos = np.array([-7, -1, 5000, 50], dtype=np.int32)
    got = host(sma.topk_select(dev(sc), dev(pos), top_k))
    assert np.all(got[0] == -1) and np.all(got[1] == -1)
    assert np.array_equal(got[2], oracle.topk_row(sc[2], top_k))
    assert np.array_equal(got[3], oracle.topk_row(sc[3, :51], top_k))


@pytest.mark.parametrize("kind", ["normal", "ties", "nan"])
def test_topk_many_long_rows(kind):
    """Rows longer than 65,536 scores, enough of them to fill the device (the
    one-workgroup-per-row path with 32-bit positions); rows checked on a
    spread sample."""
    n_rows, n_k, top_k = 1100, 70000, 2048
    sc = synth.random_scores(11 + len(kind), n_rows, n_k, kind)
    pos = _positions(n_rows, n_k, top_k, 5)
    pos[-4:] = [n_k - 1, n_k - 2, 65536, 65535]
    got = host(sma.topk_select(dev(sc), dev(pos), top_k))
    for r in list(range(0, n_rows, 37)) + list(range(n_rows - 4, n_rows)):
        ref = oracle.topk_row(sc[r, : pos[r] + 1], top_k)
        assert np.array_equal(got[r], ref), (kind, r, pos[r])


def _sampled_positions(n, n_samples=2048, cluster=16):
    """Positions the filtered top-k samples in a row of n scores (n <= 65,536):
    n_samples / 16 clusters of 16 consecutive scores whose starts are spread
    evenly over the row (rounded down to a multiple of 4)."""
    k = n_samples // cluster
    starts = [((c * (n - cluster)) // (k - 1)) & ~3 for c in range(k)]
    return np.unique(np.concatenate([np.arange(s, s + cluster) for s in starts]))


def test_topk_misleading_sample():
    """Rows whose sample misleads the filtered pass's threshold: every
    unsampled score lies above all sampled ones (far more than the 5,120 LDS
    slots are kept: the overflow slots absorb the excess and the row is redone
    by the streaming selection), or the samples hold the largest scores (fewer
    than K kept, redone too).  Both stay exact."""
    n_k, top_k = 60000, 2048
    rng = np.random.default_rng(17)
    sc = rng.random((4, n_k)).astype(np.float32)
    samp = _sampled_positions(n_k)
    rest = np.setdiff1d(np.arange(n_k), samp)
    sc[0, rest] += 10.0          # threshold far too low
    sc[1, samp] += 10.0          # threshold far too high
    sc[2, rest[::3]] += 10.0     # ~19,000 kept
    sc[3, :] = rng.random(n_k)   # an ordinary row beside them
    pos = np.array([n_k - 1, n_k - 1, n_k - 3, 40001], dtype=np.int32)
    got = host(sma.topk_select(dev(sc), dev(pos), top_k))
    for r in range(4):
        assert np.array_equal(got[r], oracle.topk_row(sc[r, : pos[r] + 1], top_k)), r


def _long_sampled_positions(n, n_clusters=1024, cluster=16):
    """Positions the split top-k samples in a row of n > 8,192 scores: 1,024
    clusters of 16 consecutive scores whose starts are spread evenly over the
    row (rounded down to a multiple of 4)."""
    starts = [((c * (n - cluster)) // (n_clusters - 1)) & ~3 for c in range(n_clusters)]
    return np.unique(np.concatenate([np.arange(s, s + cluster) for s in starts]))


@pytest.mark.parametrize("kind", ["normal", "ties", "nan_heavy"])
def test_topk_few_very_long_rows(kind):
    """A decode-shaped batch: 16 rows of up to 1,048,576 scores, too few to
    fill the device one per workgroup (the split path: one sampled threshold
    per row, one filtering pass by 16,384-score chunks, the exact selection
    over what was kept).  Ties and NaN-heavy rows keep too many or too few
    and are redone by the streaming selection."""
    n_rows, n_k, top_k = 16, 1 << 20, 2048
    sc = synth.random_scores(31 + len(kind), n_rows, n_k, kind)
    rng = np.random.default_rng(9)
    pos = rng.integers(900_000, n_k, size=n_rows).astype(np.int32)
    pos[:6] = [n_k - 1, 8191, 8192, 2047, 16383, 16384]
    got = host(sma.topk_select(dev(sc), dev(pos), top_k))
    for r in range(n_rows):
        assert np.array_equal(got[r], oracle.topk_row(sc[r, : pos[r] + 1], top_k)), (kind, r, pos[r])


def test_topk_long_misleading_sample():
    """Long rows whose sample misleads the split path's threshold: every
    unsampled score above all sampled ones (far more than 8,192 kept), the
    samples holding the largest scores (fewer than K kept), 4,500 unsampled
    scores of one chunk raised (that chunk keeps more than its 4,096-entry
    list while the row keeps fewer than 8,192), beside an ordinary row.  Each
    is redone by the streaming selection or selected exactly."""
    n_k, top_k = 200000, 2048
    rng = np.random.default_rng(23)
    sc = rng.random((4, n_k)).astype(np.float32)
    samp = _long_sampled_positions(n_k)
    rest = np.setdiff1d(np.arange(n_k), samp)
    sc[0, rest] += 10.0
    sc[1, samp] += 10.0
    chunk3 = rest[(rest >= 3 * 16384) & (rest < 4 * 16384)]
    sc[2, chunk3[:4500]] += 10.0
    pos = np.array([n_k - 1, n_k - 1, n_k - 1, 150001], dtype=np.int32)
    got = host(sma.topk_select(dev(sc), dev(pos), top_k))
    for r in range(4):
        assert np.array_equal(got[r], oracle.topk_row(sc[r, : pos[r] + 1], top_k)), r
