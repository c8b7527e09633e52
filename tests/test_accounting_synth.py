"""The accounting module against the figures the pages print, and the
seeded generator's determinism (no GPU)."""
import json
import os

import numpy as np
import pytest

from sparse_mla_attention_index_amd import accounting, synth

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_figures.json")))


def g(key):
    return GOLD[key]["value"]


def test_footnote1_per_row_figures():
    assert accounting.mla_flops_per_head_row() == g("mla_flops_per_head_row")
    assert accounting.mla_qo_bytes_per_head() == g("mla_qo_bytes_per_head")
    rows = g("rows_per_query")
    assert round(rows * (g("row_bytes_fp8_ds_mla") + 4) / 1e6, 2) == g("gather_mb_per_query")


def test_footnote1_intensity_tp8_vs_pcp():
    f8, b8, i8 = accounting.mla_query_intensity(8)
    f64, b64, i64 = accounting.mla_query_intensity(64)
    assert round(f8 / 1e6, 1) == g("tp8_mflops") and round(b8 / 1e6, 2) == g("tp8_mb")
    assert round(i8) == g("tp8_flops_per_byte")
    assert round(f64 / 1e6) == g("pcp_mflops") and round(b64 / 1e6, 2) == g("pcp_mb")
    assert round(i64) == g("pcp_flops_per_byte")


def test_footnote2_ridge():
    assert round(accounting.ridge(g("h200_tflops_bf16_dense"), g("h200_tbs"))) == g("h200_ridge")


def test_footnote3_kv_budget():
    b = accounting.glm_kv_bytes_per_token()
    assert b == g("glm_kv_bytes_per_token")
    assert 128 + 4 == g("indexer_key_bytes")
    gib = b * g("glm_1m_tokens") / 2 ** 30
    assert round(gib, 1) == g("glm_1m_gib")
    assert round(gib / 8, 1) == g("glm_1m_gib_per_gpu_dcp8")


def test_deepseek_latent_bytes():
    assert accounting.deepseek_latent_bytes_per_token(g("deepseek_layers")) == g("deepseek_bytes_per_token")


def test_workload_counts():
    pos = np.arange(65536)
    assert accounting.causal_pairs(pos) == 2_147_516_416
    assert accounting.selected_rows(pos, 2048) == 132_121_600
    assert accounting.causal_pairs(np.arange(512)) == 131_328
    assert accounting.selected_rows(np.arange(512), 128) == 57_408


@pytest.mark.parametrize("tensor", ["q_idx", "k_idx", "w", "q", "kv"])
def test_generator_subrange_consistent(tensor):
    w = synth.workload(2)
    full = synth.rows(w, tensor, 0, 80)
    part = synth.rows(w, tensor, 33, 71)
    assert np.array_equal(full[33:71], part)
    again = synth.rows(w, tensor, 0, 80)
    assert np.array_equal(full, again)


def test_generator_tiny_recipe():
    w = synth.workload(1)
    q = synth.rows(w, "q_idx", 0, 512)
    vals = np.unique((q.astype(np.uint32) << 16).view(np.float32))
    assert set(vals.tolist()) <= set(range(-3, 4))
    wt = synth.rows(w, "w", 0, 512)
    assert np.all(wt * 16 == np.round(wt * 16)) and wt.min() >= 0 and wt.max() <= 1


def test_query_positions():
    assert np.array_equal(synth.query_positions(synth.workload(1)), np.arange(512))
    p4 = synth.query_positions(synth.workload(4), rank=7)
    assert p4[0] == 7 * 8192 and p4[8192] == 8 * 8192 and p4.size == 16384
    p5 = synth.query_positions(synth.workload(5))
    assert p5.size == 64 and p5.min() >= 900_000 and p5.max() <= 1_048_575


def test_flop_crossover_against_closed_form():
    # Past top_k the causal sums have closed forms: indexer L(L+1)/2 pairs of
    # 2 H_I d_I FLOPs, attention K(K+1)/2 + (L - K) K rows of 64 (2*576 +
    # 2*512) FLOPs.  The helper's answer is the first L where the first
    # reaches the second; without the first K queries' ramp the crossover
    # would be 2 * 139,264 * K / (2 H_I d_I) = 34,816 for the 64 x 128
    # indexer and K = 2,048.
    def gap(L, h, d, k):
        return L * (L + 1) // 2 * 2 * h * d - (k * (k + 1) // 2 + (L - k) * k) * 64 * (2 * 576 + 2 * 512)

    for h, d, k in ((64, 128, 2048), (8, 64, 128), (64, 128, 512)):
        L = accounting.flop_crossover_tokens(h, d, k)
        assert L > k
        assert gap(L, h, d, k) >= 0 > gap(L - 1, h, d, k)
    approx = 2 * 64 * (2 * 576 + 2 * 512) * 2048 // (2 * 64 * 128)
    assert approx == 34816
    assert abs(accounting.flop_crossover_tokens(64, 128, 2048) - approx) < 0.04 * approx
