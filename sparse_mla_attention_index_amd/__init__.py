"""MI355X (gfx950) sparse-MLA prefill path: indexer scores -> per-query
top-k -> sparse MLA over the selected latent rows, plus one PCP rank's
share, one DCP rank's partial attention with the log-sum-exp merge, and the
FP8 indexer (per-row FP8 quantisation, e4m3 x e4m3 scores) and the
absorption products around sparse MLA.  The compute
runs in hand-written HIP kernels behind the C ABI of include/sma.h
(libsma.so); this package is the thin Python binding."""
from ._lib import (SmaError, absorb_q, dcp_shard_partial, dcp_shard_partial_noalloc, dense_mha_prefill, index_scores, index_scores_fp8, last_error, lib,  # noqa: F401
                   lse_merge, pcp_rank_share, prefill, prefill_fp8_indexer, quantize_fp8_rows,
                   project_out, sparse_mla_prefill, topk_select, version, workspace_bytes)
