"""Pins for the PCP rank share and the FP8 storage decode (no GPU).

PCP (GLM-5.3 part 2, "PCP : répartir les tokens, pas les têtes"): 16 chunks,
each of 8 ranks takes one early and one late chunk.  The union of the 8
shares must equal the unsharded prefill bit for bit, and the causal work per
rank is the closed form 16*C^2 + C pairs for every rank.

FP8 (footnote 3 of the same page: 128 FP8 values plus a 4-byte scale): the
oracle's e4m3fn table is compared with torch's float8_e4m3fn cast.
"""
import numpy as np
import pytest
import torch

import oracle
from sparse_mla_attention_index_amd import accounting, synth

TAU = 1.0 / np.sqrt(192.0)


def test_pcp_positions_pairing():
    L = 131072
    c = L // 16
    for r in range(8):
        pos = oracle.pcp_positions(r, 8, L)
        assert pos.size == 2 * c
        assert pos[0] == r * c and pos[c - 1] == (r + 1) * c - 1
        assert pos[c] == (15 - r) * c and pos[-1] == (16 - r) * c - 1
    allpos = np.concatenate([oracle.pcp_positions(r, 8, L) for r in range(8)])
    assert np.array_equal(np.sort(allpos), np.arange(L))


def test_pcp_balance_closed_form():
    L, K = 131072, 2048
    c = L // 16
    for r in range(8):
        pos = oracle.pcp_positions(r, 8, L)
        assert accounting.causal_pairs(pos) == 16 * c * c + c == 1_073_750_016
    assert accounting.selected_rows(oracle.pcp_positions(0, 8, L), K) == 31_458_304
    for r in range(1, 8):
        assert accounting.selected_rows(oracle.pcp_positions(r, 8, L), K) == 33_554_432


def test_pcp_union_equals_unsharded():
    rng = np.random.default_rng(9)
    L, P, K = 192, 4, 24
    q_idx = rng.integers(-3, 4, size=(L, 4, 8)).astype(np.float64)
    k_idx = rng.integers(-3, 4, size=(L, 8)).astype(np.float64)
    w = np.round(rng.random((L, 4)) * 16) / 16
    q = rng.standard_normal((L, 64, 576)) * 0.1
    kv = rng.standard_normal((L, 576)) * 0.1
    _, idx_full, out_full, lse_full = oracle.prefill(q_idx, w, k_idx, q, kv, np.arange(L), K, TAU)
    seen = np.zeros(L, bool)
    for r in range(P):
        pos = oracle.pcp_positions(r, P, L)
        _, idx, out, lse = oracle.pcp_rank_share(r, P, q_idx, w, k_idx, q, kv, K, TAU)
        assert np.array_equal(idx, idx_full[pos])
        assert np.array_equal(out, out_full[pos]) and np.array_equal(lse, lse_full[pos])
        seen[pos] = True
    assert seen.all()


def test_e4m3fn_table_matches_torch():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = oracle.e4m3fn_table()
    nan = np.isnan(t)
    assert np.array_equal(nan, np.isnan(mine)) and nan.sum() == 2
    assert np.array_equal(t[~nan], mine[~nan])
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9


def test_fp8_values_exact_in_bf16():
    vals = oracle.e4m3fn_table()
    vals = vals[~np.isnan(vals)]
    back = torch.from_numpy(vals).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(back, vals)


def test_fp8_dequant_per_token():
    codes = np.array([[0x38, 0xB8, 0x00], [0x40, 0x7E, 0x01]], dtype=np.uint8)  # 1, -1, 0 / 2, 448, 2^-9
    scale = np.array([0.5, 2.0], dtype=np.float32)
    x = oracle.fp8_rows_to_f64(codes, scale)
    assert x.tolist() == [[0.5, -0.5, 0.0], [4.0, 896.0, 2.0 ** -8]]


def test_fp8_generator_roundtrip():
    """The decode workload's FP8 rows dequantise to within e4m3's half-ulp
    (2^-4 relative) of the drawn values, and max |x| maps to 448."""
    w = synth.workload(5)
    codes, scale = synth.rows(w, "kv", 1000, 1004)
    x32 = synth._gen_f32_rows(w, "kv", 1000, 1004)
    deq = oracle.fp8_rows_to_f64(codes, scale)
    assert np.all(np.abs(deq - x32) <= np.abs(x32) * 2.0 ** -4 + scale[:, None] * 2.0 ** -9 + 1e-12)
    assert np.all(np.abs(oracle.e4m3fn_table()[codes]).max(axis=1) == 448.0)


# --------------------------------------------- fp8_ds_mla (656-byte rows) --

def test_fp8_ds_mla_layout_markers():
    """A row built byte by byte: codes 0x38 (= 1.0) everywhere, scales
    1, 2, 4, 8, rope bf16 0.5 (0x3F00) -> dims 0..127 = 1, 128..255 = 2,
    256..383 = 4, 384..511 = 8, 512..575 = 0.5."""
    row = np.zeros((1, 656), np.uint8)
    row[0, :512] = 0x38
    row[0, 512:528] = np.array([1, 2, 4, 8], "<f4").view(np.uint8)
    row[0, 528:] = np.full(64, 0x3F00, "<u2").view(np.uint8)
    x = oracle.fp8_ds_mla_rows_to_f64(row)[0]
    assert np.array_equal(x, np.concatenate([np.full(128, 1.0), np.full(128, 2.0), np.full(128, 4.0),
                                             np.full(128, 8.0), np.full(64, 0.5)]))


def test_fp8_ds_mla_decode_of_torch_packed_rows():
    """Rows packed here with torch's casts (codes per 128-dim block, its
    scale, bf16 rope) decode to e4m3(code)*scale and the bf16 rope exactly,
    within the format's half-spacing of the fp32 source."""
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((40, 576)) * np.exp2(rng.integers(-6, 6, (40, 1)))).astype(np.float32)
    x[3, 128:256] = 0.0                                   # an all-zero block: scale 0
    rows = np.zeros((40, 656), np.uint8)
    dec_ref = np.zeros((40, 576))
    for b in range(4):
        blk = x[:, 128 * b:128 * (b + 1)]
        s = (np.abs(blk).max(axis=1) / np.float32(448)).astype(np.float32)
        safe = np.where(s > 0, s, 1).astype(np.float32)
        c = torch.from_numpy(np.clip(blk / safe[:, None], -448, 448).astype(np.float32)).to(torch.float8_e4m3fn)
        rows[:, 128 * b:128 * (b + 1)] = c.view(torch.uint8).numpy()
        rows[:, 512 + 4 * b:516 + 4 * b] = s.astype("<f4").view(np.uint8).reshape(40, 4)
        dec_ref[:, 128 * b:128 * (b + 1)] = c.to(torch.float64).numpy() * s.astype(np.float64)[:, None]
    rb = torch.from_numpy(x[:, 512:]).to(torch.bfloat16)
    rows[:, 528:] = rb.view(torch.int16).numpy().view(np.uint8).reshape(40, 128)
    dec_ref[:, 512:] = rb.to(torch.float64).numpy()
    got = oracle.fp8_ds_mla_rows_to_f64(rows)
    assert np.array_equal(got, dec_ref)
    assert np.all(got[3, 128:256] == 0)
    err = np.abs(got[:, :512] - x[:, :512])
    bound = np.repeat(np.abs(x[:, :512]).reshape(40, 4, 128).max(axis=2) / 448, 128, axis=1)
    assert np.all(err <= (2.0 ** -4 * np.abs(x[:, :512]) + 2.0 ** -10 * bound) * (1 + 1e-6))
    # the input generator's packer gives the same bytes
    assert np.array_equal(synth.to_fp8_ds_mla_rows(x), rows)


def test_fp8_ds_mla_rejects_other_shapes():
    with pytest.raises(ValueError):
        oracle.fp8_ds_mla_rows_to_f64(np.zeros((2, 580), np.uint8))
