"""MI355X (gfx950) sparse-MLA prefill path: indexer scores -> per-query
top-k -> sparse MLA over the selected latent rows, plus one PCP rank's
share.  The compute runs in hand-written HIP kernels behind the C ABI of
include/sma.h (libsma.so); this package is the thin Python binding."""
from ._lib import (SmaError, index_scores, last_error, lib, pcp_rank_share, prefill,  # noqa: F401
                   sparse_mla_prefill, topk_select, version, workspace_bytes)
