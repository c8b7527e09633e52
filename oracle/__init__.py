"""CPU oracle (test infrastructure only; see sma_oracle's header)."""
from .sma_oracle import *  # noqa: F401,F403
from .sma_oracle import (bf16_bits_to_f64, e4m3fn_table, fp8_rows_to_f64, index_scores,  # noqa: F401
                         topk_row, topk_select, topk_threshold, sparse_mla, prefill,
                         pcp_positions, pcp_rank_share, keys_f64, dcp_shard_rows, dcp_shard_partial,
                         lse_merge, e4m3fn_encode, quantize_fp8_rows, index_scores_fp8,
                         fp8_ds_mla_rows_to_f64, DS_ROW_BYTES,
                         absorb_q, project_out, dense_mha_prefill)
