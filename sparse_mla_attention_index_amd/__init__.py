"""MI355X (gfx950) sparse-MLA prefill path: indexer scores -> per-query
top-k -> sparse MLA over the selected latent rows, plus one PCP rank's
share and one DCP rank's partial attention with the log-sum-exp merge.  The compute runs in hand-written HIP kernels behind the C ABI of
include/sma.h (libsma.so); this package is the thin Python binding."""
from ._lib import (SmaError, dcp_shard_partial, index_scores, last_error, lib, lse_merge,  # noqa: F401
                   pcp_rank_share, prefill, sparse_mla_prefill, topk_select, version, workspace_bytes)
