"""Pins of the oracle's FP8-query indexer (no GPU).

The e4m3fn encoder is checked against torch's float8_e4m3fn cast (a library
routine written independently of the oracle) on every code, every midpoint
between neighbouring codes and the fp32 values either side of it, and on
random values over the whole range; the row quantiser against the same cast
and the format's error bound; the FP8 indexer against exact rational brute
force on tiny inputs with distinct per-(query, head) and per-key scales.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle as O


def torch_codes(y) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def torch_values(codes) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


FINITE = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)


def test_encode_every_code_roundtrips():
    vals = torch_values(FINITE)
    assert np.array_equal(O.e4m3fn_encode(vals), FINITE)   # -0.0 keeps code 0x80


def test_encode_midpoints_ties_to_even():
    pos = np.sort(torch_values(FINITE[FINITE < 0x80]))      # 0 .. 448, 127 values
    mid = (pos[:-1] + pos[1:]) / 2                           # exact in fp32 (5 significant bits)
    m32 = mid.astype(np.float32)
    assert np.array_equal(m32.astype(np.float64), mid)
    lo = np.nextafter(m32, np.float32(0))
    hi = np.nextafter(m32, np.float32(np.inf))
    for y in (m32, lo, hi, -m32, -lo, -hi):
        assert np.array_equal(O.e4m3fn_encode(y), torch_codes(y))
    # a tie goes to the code with an even mantissa
    assert np.all(O.e4m3fn_encode(m32) % 2 == 0)
    # half the smallest subnormal rounds to zero, just above it to 2^-9
    assert O.e4m3fn_encode(np.float32(2.0 ** -10)) == 0
    assert O.e4m3fn_encode(np.nextafter(np.float32(2.0 ** -10), np.float32(1))) == 1


def test_encode_random_values_match_torch():
    rng = np.random.default_rng(7)
    mag = np.exp2(rng.uniform(-14.0, np.log2(448.0), 200_000)).astype(np.float32)
    y = np.where(rng.random(mag.size) < 0.5, -mag, mag).astype(np.float32)
    y = np.clip(y, -448, 448)
    assert np.array_equal(O.e4m3fn_encode(y), torch_codes(y))


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        O.e4m3fn_encode(np.array([449.0]))


def test_quantize_rows_against_torch_cast():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((300, 128)).astype(np.float32) * np.exp2(rng.integers(-20, 20, (300, 1)))
    x = x.astype(np.float32)
    codes, scale = O.quantize_fp8_rows(x)
    amax = np.abs(x).max(axis=1)
    s_ref = (amax / np.float32(448.0)).astype(np.float32)
    assert np.array_equal(scale, s_ref)
    y = np.clip(x / s_ref[:, None], -448, 448).astype(np.float32)
    assert np.array_equal(codes, torch_codes(y))


def test_quantize_rows_properties():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((200, 64)).astype(np.float32)
    x[5] = 0.0
    x[6, 3] = -7.5                         # a row whose amax element is negative
    codes, scale = O.quantize_fp8_rows(x)
    assert scale[5] == 0 and not codes[5].any()
    v = torch_values(codes)
    for r in range(x.shape[0]):
        if r == 5:
            continue
        # the row's largest element lands on +-448 (codes 0x7E / 0xFE)
        j = np.argmax(np.abs(x[r]))
        assert codes[r, j] & 0x7F == 0x7E and np.signbit(v[r, j]) == np.signbit(x[r, j])
        # round-to-nearest error of the format: half a spacing, relative 2^-4
        # in the normal range and 2^-10 absolute among the subnormals
        y = x[r].astype(np.float64) / scale[r]
        err = np.abs(y - v[r])
        assert np.all(err <= (2.0 ** -4 * np.abs(y) + 2.0 ** -10) * (1 + 1e-6))


def _bruteforce_fp8_scores(q8, qs, w, k8, ks, pos):
    """Exact rationals: values from torch's cast, scales and weights as
    Fractions, ReLU and the head sum written out."""
    qv = torch_values(q8)
    kv = torch_values(k8)
    out = []
    for i in range(q8.shape[0]):
        row = []
        for s in range(int(pos[i]) + 1):
            tot = Fraction(0)
            for h in range(q8.shape[1]):
                dot = sum(Fraction(float(qv[i, h, d])) * Fraction(float(kv[s, d])) for d in range(q8.shape[2]))
                x = dot * Fraction(float(qs[i, h])) * Fraction(float(ks[s]))
                if x > 0:
                    tot += Fraction(float(w[i, h])) * x
            row.append(tot)
        out.append(row)
    return out


def test_index_scores_fp8_bruteforce():
    rng = np.random.default_rng(13)
    n_q, H, D, n_k = 3, 4, 16, 9
    q8 = rng.choice(FINITE, size=(n_q, H, D)).astype(np.uint8)
    k8 = rng.choice(FINITE, size=(n_k, D)).astype(np.uint8)
    qs = np.exp2(rng.integers(-4, 4, (n_q, H))).astype(np.float32) * rng.choice([1.0, 1.5, 0.75], (n_q, H))
    ks = np.exp2(rng.integers(-4, 4, n_k)).astype(np.float32) * rng.choice([1.0, 1.25], n_k)
    w = (rng.integers(-16, 17, (n_q, H)) / 16.0).astype(np.float32)
    pos = np.array([0, 4, 8], dtype=np.int32)
    got = O.index_scores_fp8(q8, qs.astype(np.float32), w, k8, ks.astype(np.float32), pos)
    ref = _bruteforce_fp8_scores(q8, qs, w, k8, ks, pos)
    for g, r in zip(got, ref):
        assert len(g) == len(r)
        for a, b in zip(g, r):
            assert abs(Fraction(float(a)) - b) <= abs(b) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def test_index_scores_fp8_scale_placement():
    """Doubling one head's q scale doubles only that head's ReLU term;
    doubling one key's scale doubles only that key's score."""
    rng = np.random.default_rng(14)
    q8 = rng.choice(FINITE, size=(2, 4, 16)).astype(np.uint8)
    k8 = rng.choice(FINITE, size=(6, 16)).astype(np.uint8)
    qs = np.ones((2, 4), np.float32)
    ks = np.ones(6, np.float32)
    w = np.ones((2, 4), np.float32)
    pos = np.array([5, 5], np.int32)
    base = O.index_scores_fp8(q8, qs, w, k8, ks, pos)
    ks2 = ks.copy()
    ks2[3] = 2
    s2 = O.index_scores_fp8(q8, qs, w, k8, ks2, pos)
    for b, c in zip(base, s2):
        assert np.allclose(np.delete(c, 3), np.delete(b, 3), rtol=0, atol=0) and c[3] == 2 * b[3]
    qs2 = qs.copy()
    qs2[1, 2] = 2
    s3 = O.index_scores_fp8(q8, qs2, w, k8, ks, pos)
    assert np.array_equal(s3[0], base[0])
    w_only = np.zeros((2, 4), np.float32)
    w_only[1, 2] = 1
    head = O.index_scores_fp8(q8, qs, w_only, k8, ks, pos)[1]
    assert np.allclose(s3[1], base[1] + head, rtol=1e-12, atol=0)


def test_fp8_queries_perturb_scores():
    """On the 64 x 128 N(0,1) indexer shape the FP8 query rows move scores by
    about the format's 2^-4 half-spacing, well past 1e-3 of the score scale:
    the FP8 path is compared with the oracle on the same FP8 codes, not with
    the bf16 path."""
    rng = np.random.default_rng(15)
    q = rng.standard_normal((4, 64, 128)).astype(np.float32)
    k = rng.standard_normal((256, 128)).astype(np.float32)
    w = rng.uniform(0, 1, (4, 64)).astype(np.float32) / 8
    pos = np.full(4, 255, np.int32)
    q8, qs = O.quantize_fp8_rows(q.reshape(-1, 128))
    k8, ks = O.quantize_fp8_rows(k)
    exact = O.index_scores(q.astype(np.float64), w.astype(np.float64), k.astype(np.float64), pos)
    f8 = O.index_scores_fp8(q8.reshape(4, 64, 128), qs.reshape(4, 64), w, k8, ks, pos)
    rel = max(np.max(np.abs(a - b)) / np.max(np.abs(b)) for a, b in zip(f8, exact))
    assert 1e-3 < rel < 0.1
