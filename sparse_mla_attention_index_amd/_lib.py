"""ctypes binding of libsma.so (the HIP kernels behind include/sma.h).

Argument marshalling only: every step of the path runs in the library's
kernels.  Tensors are torch tensors on one ROCm device; bf16 data may be
passed as torch.bfloat16 or as 16-bit integer bit patterns, FP8 data as
torch.float8_e4m3fn or uint8 codes.  Work is enqueued on torch's current
stream of the tensors' device.  Any failure raises SmaError carrying the
library's message; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsma.so")
# the debug build (device-resident range checks, workspace fill; include/sma.h)
DEBUG_LIB_PATH = os.path.join(_HERE, "libsma_debug.so")
SMA_BUILD_DEBUG_CHECKS = 1

SMA_DT_BF16, SMA_DT_FP8_E4M3, SMA_DT_FP32, SMA_DT_FP8_DS_MLA = 0, 1, 2, 3
DS_ROW_BYTES = 656   # fp8_ds_mla latent row: 512 e4m3 codes, 4 fp32 scales, 64 bf16 rope dims
SMA_OP_INDEX_SCORES, SMA_OP_TOPK, SMA_OP_SPARSE_MLA, SMA_OP_PREFILL, SMA_OP_PCP_SHARE = 0, 1, 2, 3, 4
SMA_OP_DCP_PARTIAL, SMA_OP_DENSE_MHA = 5, 6
HEADS, D_QK, D_V = 64, 576, 512

# (name, restype, argtypes) of every entry point declared in include/sma.h
_P, _I32, _I64, _SZ, _F = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
SIGNATURES = {
    "sma_index_scores": (_I32, [_P, _P, _I64, _P, _P, _I32, _P, _I32, _I64, _I32, _I32, _P, _I64, _P]),
    "sma_topk_select": (_I32, [_P, _I64, _P, _I32, _I64, _I32, _P, _P, _SZ, _P]),
    "sma_sparse_mla_prefill": (_I32, [_P, _P, _P, _I32, _I64, _P, _I32, _I32, _F, _P, _I32, _P, _P, _SZ, _P]),
    "sma_prefill": (_I32, [_P, _P, _I64, _P, _P, _I32, _P, _P, _P, _I32, _P, _I32, _I64, _I32, _I32, _I32, _F,
                           _P, _I32, _P, _P, _P, _SZ, _P]),
    "sma_pcp_rank_share": (_I32, [_I32, _I32, _I64, _P, _P, _I64, _P, _P, _I32, _P, _P, _P, _I32, _I32, _I32,
                                  _I32, _F, _P, _I32, _P, _P, _P, _SZ, _P]),
    "sma_dcp_shard_partial": (_I32, [_I32, _I32, _P, _P, _P, _I32, _I64, _P, _I32, _I32, _F, _P, _P, _P, _SZ,
                                     _P]),
    "sma_dcp_shard_partial_noalloc": (_I32, [_I32, _I32, _P, _P, _P, _I32, _I64, _P, _I32, _I32, _F, _P, _P, _P]),
    "sma_dense_mha_prefill": (_I32, [_P, _P, _P, _P, _P, _I32, _I64, _F, _P, _I32, _P, _P, _SZ, _P]),
    "sma_lse_merge": (_I32, [_P, _P, _I32, _I32, _P, _I32, _P, _P]),
    "sma_quantize_fp8_rows": (_I32, [_P, _I64, _I32, _P, _P, _P]),
    "sma_absorb_q": (_I32, [_P, _P, _I32, _I32, _P, _I64, _P]),
    "sma_project_out": (_I32, [_P, _P, _I32, _I32, _P, _P]),
    "sma_index_scores_fp8": (_I32, [_P, _P, _P, _I64, _P, _P, _P, _I32, _I64, _I32, _I32, _P, _I64, _P]),
    "sma_prefill_fp8_indexer": (_I32, [_P, _P, _P, _I64, _P, _P, _P, _P, _P, _I32, _P, _I32, _I64, _I32, _I32,
                                       _I32, _F, _P, _I32, _P, _P, _P, _SZ, _P]),
    "sma_workspace_bytes": (_SZ, [_I32, _I32, _I64, _I32, _I32, _I32]),
    "sma_last_error": (ctypes.c_char_p, []),
    "sma_version": (_I32, []),
    "sma_build_flags": (_I32, []),
}

_lib = None


class SmaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"sma status {status}: {msg}")
        self.status = status


def load(path: str):
    """Open one build of the library with every entry point's signature set
    (raises if it was not built: there is no fallback)."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing; build it with `python -m sparse_mla_attention_index_amd.build`")
    L = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    return L


def lib():
    """The library every wrapper below calls: libsma.so, or the debug build
    when SMA_DEBUG_LIBRARY=1 is set before the first call."""
    global _lib
    if _lib is None:
        _lib = load(DEBUG_LIB_PATH if os.environ.get("SMA_DEBUG_LIBRARY") == "1" else LIB_PATH)
    return _lib


class debug_library:
    """Context manager: the wrappers call the debug build inside the block
    and the library they called before it afterwards."""

    def __enter__(self):
        global _lib
        self._prev = lib()
        _lib = load(DEBUG_LIB_PATH)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self._prev
        return False


def build_flags() -> int:
    return int(lib().sma_build_flags())


def last_error() -> str:
    return lib().sma_last_error().decode()


def version() -> int:
    return int(lib().sma_version())


def workspace_bytes(op: int, n_q: int, n_k: int, top_k: int, h_idx: int = 64, d_idx: int = 128) -> int:
    return int(lib().sma_workspace_bytes(op, n_q, n_k, top_k, h_idx, d_idx))


def _check(status: int):
    if status != 0:
        raise SmaError(status, last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _bf16(t, name):
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name}: expected bf16 data (bfloat16 or 16-bit bit patterns), got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _keys(t, scale, name):
    """-> dtype code for a key/KV tensor: bf16, FP8 codes + per-row scale, or
    (uint8 [n, 656] with no scale) fp8_ds_mla latent rows."""
    if t.dtype == torch.uint8 and scale is None and t.dim() == 2 and t.shape[1] == DS_ROW_BYTES:
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        return SMA_DT_FP8_DS_MLA
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        if scale is None or scale.dtype != torch.float32 or not scale.is_contiguous():
            raise ValueError(f"{name}: FP8 data needs a contiguous fp32 per-row scale")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        return SMA_DT_FP8_E4M3
    _bf16(t, name)
    if scale is not None:
        raise ValueError(f"{name}: a scale is only taken with FP8 data")
    return SMA_DT_BF16


def _w_stride(w, n_q, h):
    if w.dtype != torch.float32 or w.dim() != 2 or w.shape[1] != h or w.stride(1) != 1:
        raise ValueError("w must be fp32 [n_q, h_idx] with unit stride along heads")
    return int(w.stride(0)) if n_q > 1 or w.stride(0) == 0 else h


def index_scores(q_idx, w, k_idx, q_pos, *, k_scale=None, scores=None):
    """Indexer scores [n_q, n_k] fp32; only s <= q_pos[i] is written."""
    n_q, h, d = q_idx.shape
    n_k = k_idx.shape[0]
    _bf16(q_idx, "q_idx")
    kdt = _keys(k_idx, k_scale, "k_idx")
    if q_pos.dtype != torch.int32 or not q_pos.is_contiguous():
        raise ValueError("q_pos must be contiguous int32")
    if scores is None:
        scores = torch.empty((n_q, n_k), dtype=torch.float32, device=q_idx.device)
    if scores.dtype != torch.float32 or scores.stride(1) != 1:
        raise ValueError("scores must be fp32 with unit column stride")
    _check(lib().sma_index_scores(_ptr(q_idx), _ptr(w), _w_stride(w, n_q, h), _ptr(k_idx), _ptr(k_scale), kdt,
                                  _ptr(q_pos), n_q, n_k, h, d, _ptr(scores), scores.stride(0),
                                  _stream(q_idx.device)))
    return scores


def _fp8(t, name):
    if t.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise TypeError(f"{name}: expected e4m3fn codes (float8_e4m3fn or uint8), got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _f32(t, name):
    if t is None or t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous fp32 tensor")


def quantize_fp8_rows(x, *, codes=None, scale=None):
    """Per-row FP8: x bf16 [..., d] (d = 64 or 128) -> (codes uint8 [..., d],
    scale fp32 [...]) with scale = amax/448 and nearest-even e4m3fn codes."""
    _bf16(x, "x")
    d = x.shape[-1]
    n_rows = x.numel() // d if d else 0
    if codes is None:
        codes = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    _fp8(codes, "codes")
    _f32(scale, "scale")
    if codes.numel() != x.numel() or scale.numel() != n_rows:
        raise ValueError("codes / scale sizes do not match x")
    _check(lib().sma_quantize_fp8_rows(_ptr(x), n_rows, d, _ptr(codes), _ptr(scale), _stream(x.device)))
    return codes, scale


def index_scores_fp8(q_idx, q_scale, w, k_idx, k_scale, q_pos, *, scores=None):
    """Indexer scores [n_q, n_k] fp32 from FP8 queries [n_q, 64, 128] with
    per-(query, head) scales [n_q, 64] and FP8 keys [n_k, 128] with per-key
    scales; only s <= q_pos[i] is written."""
    n_q, h, d = q_idx.shape
    n_k = k_idx.shape[0]
    _fp8(q_idx, "q_idx")
    _fp8(k_idx, "k_idx")
    _f32(q_scale, "q_scale")
    _f32(k_scale, "k_scale")
    if q_pos.dtype != torch.int32 or not q_pos.is_contiguous():
        raise ValueError("q_pos must be contiguous int32")
    if scores is None:
        scores = torch.empty((n_q, n_k), dtype=torch.float32, device=q_idx.device)
    if scores.dtype != torch.float32 or scores.stride(1) != 1:
        raise ValueError("scores must be fp32 with unit column stride")
    _check(lib().sma_index_scores_fp8(_ptr(q_idx), _ptr(q_scale), _ptr(w), _w_stride(w, n_q, h), _ptr(k_idx),
                                      _ptr(k_scale), _ptr(q_pos), n_q, n_k, h, d, _ptr(scores), scores.stride(0),
                                      _stream(q_idx.device)))
    return scores


def topk_select(scores, q_pos, top_k: int, *, n_k: int | None = None, idx=None, workspace=None):
    """Top-k positions per row, ascending, -1 padded: int32 [n_q, top_k].

    `workspace` (uint8 device tensor): rows longer than 65,536 scores are
    split across workgroups when it holds workspace_bytes(SMA_OP_TOPK, ...)
    bytes; one of that size is allocated here when none is given."""
    n_q = scores.shape[0]
    n_k = scores.shape[1] if n_k is None else n_k
    if scores.dtype != torch.float32 or scores.stride(1) != 1:
        raise ValueError("scores must be fp32 with unit column stride")
    if q_pos.dtype != torch.int32 or not q_pos.is_contiguous():
        raise ValueError("q_pos must be contiguous int32")
    if idx is None:
        idx = torch.empty((n_q, top_k), dtype=torch.int32, device=scores.device)
    if workspace is None and n_q > 0:
        nbytes = workspace_bytes(SMA_OP_TOPK, n_q, n_k, top_k)
        if nbytes > 0:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=scores.device)
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().sma_topk_select(_ptr(scores), scores.stride(0), _ptr(q_pos), n_q, n_k, top_k, _ptr(idx),
                                 _ptr(workspace), ws_n, _stream(scores.device)))
    return idx


def sparse_mla_prefill(q, kv, idx, sm_scale: float, *, kv_scale=None, out=None, out_dtype=torch.bfloat16,
                       lse=None, want_lse: bool = False, workspace=None):
    """Sparse MLA over idx: returns (out [n_q, 64, 512], lse [n_q, 64] or None).

    `workspace` (uint8 device tensor, optional): with at least
    workspace_bytes(SMA_OP_SPARSE_MLA, n_q, n_k, top_k) bytes, small
    batches split each query's rows across workgroups."""
    n_q = q.shape[0]
    _bf16(q, "q")
    kdt = _keys(kv, kv_scale, "kv")
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be contiguous int32")
    if out is None:
        out = torch.empty((n_q, HEADS, D_V), dtype=out_dtype, device=q.device)
    odt = SMA_DT_FP32 if out.dtype == torch.float32 else SMA_DT_BF16
    if lse is None and want_lse:
        lse = torch.empty((n_q, HEADS), dtype=torch.float32, device=q.device)
    ws_n = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().sma_sparse_mla_prefill(_ptr(q), _ptr(kv), _ptr(kv_scale), kdt, kv.shape[0], _ptr(idx), n_q,
                                        idx.shape[1], float(sm_scale), _ptr(out), odt, _ptr(lse),
                                        _ptr(workspace), ws_n, _stream(q.device)))
    return out, lse


def prefill(q_idx, w, k_idx, q, kv, q_pos, top_k: int, sm_scale: float, *, k_scale=None, kv_scale=None,
            out=None, out_dtype=torch.bfloat16, want_lse=False, idx_out=None, workspace=None):
    """indexer -> top-k -> sparse MLA; returns (out, lse or None, idx or None)."""
    n_q, h, d = q_idx.shape
    n_k = k_idx.shape[0]
    kdt = _keys(k_idx, k_scale, "k_idx")
    vdt = _keys(kv, kv_scale, "kv")
    _bf16(q_idx, "q_idx")
    _bf16(q, "q")
    dev = q.device
    if out is None:
        out = torch.empty((n_q, HEADS, D_V), dtype=out_dtype, device=dev)
    odt = SMA_DT_FP32 if out.dtype == torch.float32 else SMA_DT_BF16
    lse = torch.empty((n_q, HEADS), dtype=torch.float32, device=dev) if want_lse else None
    if workspace is None:
        nbytes = workspace_bytes(SMA_OP_PREFILL, n_q, n_k, top_k, h, d)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(lib().sma_prefill(_ptr(q_idx), _ptr(w), _w_stride(w, n_q, h), _ptr(k_idx), _ptr(k_scale), kdt,
                             _ptr(q), _ptr(kv), _ptr(kv_scale), vdt, _ptr(q_pos), n_q, n_k, h, d, top_k,
                             float(sm_scale), _ptr(out), odt, _ptr(lse), _ptr(idx_out), _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(dev)))
    return out, lse, idx_out


def prefill_fp8_indexer(q_idx, q_scale, w, k_idx, k_scale, q, kv, q_pos, top_k: int, sm_scale: float, *,
                        kv_scale=None, out=None, out_dtype=torch.bfloat16, want_lse=False, idx_out=None,
                        workspace=None):
    """prefill() with the FP8 indexer (FP8 queries + per-head scales, FP8
    keys + per-key scales); returns (out, lse or None, idx or None)."""
    n_q, h, d = q_idx.shape
    n_k = k_idx.shape[0]
    _fp8(q_idx, "q_idx")
    _fp8(k_idx, "k_idx")
    _f32(q_scale, "q_scale")
    _f32(k_scale, "k_scale")
    vdt = _keys(kv, kv_scale, "kv")
    _bf16(q, "q")
    dev = q.device
    if out is None:
        out = torch.empty((n_q, HEADS, D_V), dtype=out_dtype, device=dev)
    odt = SMA_DT_FP32 if out.dtype == torch.float32 else SMA_DT_BF16
    lse = torch.empty((n_q, HEADS), dtype=torch.float32, device=dev) if want_lse else None
    if workspace is None:
        nbytes = workspace_bytes(SMA_OP_PREFILL, n_q, n_k, top_k, h, d)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(lib().sma_prefill_fp8_indexer(_ptr(q_idx), _ptr(q_scale), _ptr(w), _w_stride(w, n_q, h), _ptr(k_idx),
                                         _ptr(k_scale), _ptr(q), _ptr(kv), _ptr(kv_scale), vdt, _ptr(q_pos), n_q,
                                         n_k, h, d, top_k, float(sm_scale), _ptr(out), odt, _ptr(lse),
                                         _ptr(idx_out), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(dev)))
    return out, lse, idx_out


def absorb_q(q_nope, w_uk, *, out=None):
    """q_lat[i,h,:] = W_UK[h]^T q_nope[i,h,:]: q_nope bf16 [n, H, 128], w_uk
    bf16 [H, 128, 512] -> bf16 [n, H, 512]; `out` may be a sparse-MLA query
    [n, H, 576] (its first 512 dims are written, the rope dims kept)."""
    n, heads, d = q_nope.shape
    _bf16(q_nope, "q_nope")
    _bf16(w_uk, "w_uk")
    if d != 128 or tuple(w_uk.shape) != (heads, 128, 512):
        raise ValueError("q_nope [n, H, 128] and w_uk [H, 128, 512] expected")
    if out is None:
        out = torch.empty((n, heads, 512), dtype=torch.bfloat16, device=q_nope.device)
    _bf16(out, "out")
    if out.dim() != 3 or tuple(out.shape[:2]) != (n, heads) or out.shape[2] < 512:
        raise ValueError("out must be [n, H, >= 512]")
    _check(lib().sma_absorb_q(_ptr(q_nope), _ptr(w_uk), n, heads, _ptr(out), out.shape[2], _stream(q_nope.device)))
    return out


def project_out(o_lat, w_uv, *, out=None):
    """o[i,h,:] = W_UV[h] o_lat[i,h,:]: o_lat bf16 [n, H, 512], w_uv bf16
    [H, 128, 512] -> bf16 [n, H, 128]."""
    n, heads, d = o_lat.shape
    _bf16(o_lat, "o_lat")
    _bf16(w_uv, "w_uv")
    if d != 512 or tuple(w_uv.shape) != (heads, 128, 512):
        raise ValueError("o_lat [n, H, 512] and w_uv [H, 128, 512] expected")
    if out is None:
        out = torch.empty((n, heads, 128), dtype=torch.bfloat16, device=o_lat.device)
    _bf16(out, "out")
    _check(lib().sma_project_out(_ptr(o_lat), _ptr(w_uv), n, heads, _ptr(out), _stream(o_lat.device)))
    return out


def pcp_rank_share(rank: int, pcp_size: int, q_idx_share, w_share, k_idx, q_share, kv, top_k: int,
                   sm_scale: float, *, k_scale=None, kv_scale=None, out=None, out_dtype=torch.bfloat16,
                   want_lse=False, idx_share=None, workspace=None):
    """One PCP rank's share (chunks rank and 2*pcp_size-1-rank of a prompt of
    k_idx.shape[0] tokens); returns (out, lse or None, idx or None)."""
    n_q, h, d = q_idx_share.shape
    L = k_idx.shape[0]
    kdt = _keys(k_idx, k_scale, "k_idx")
    vdt = _keys(kv, kv_scale, "kv")
    _bf16(q_idx_share, "q_idx_share")
    _bf16(q_share, "q_share")
    dev = q_share.device
    if out is None:
        out = torch.empty((n_q, HEADS, D_V), dtype=out_dtype, device=dev)
    odt = SMA_DT_FP32 if out.dtype == torch.float32 else SMA_DT_BF16
    lse = torch.empty((n_q, HEADS), dtype=torch.float32, device=dev) if want_lse else None
    if workspace is None:
        nbytes = workspace_bytes(SMA_OP_PCP_SHARE, n_q, L, top_k, h, d)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(lib().sma_pcp_rank_share(rank, pcp_size, L, _ptr(q_idx_share), _ptr(w_share),
                                    _w_stride(w_share, n_q, h), _ptr(k_idx), _ptr(k_scale), kdt, _ptr(q_share),
                                    _ptr(kv), _ptr(kv_scale), vdt, h, d, top_k, float(sm_scale), _ptr(out), odt,
                                    _ptr(lse), _ptr(idx_share), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream(dev)))
    return out, lse, idx_share


def dense_mha_prefill(q, kv, w_uk, w_uv, q_pos, sm_scale: float, *, out=None, out_dtype=torch.bfloat16,
                      want_lse: bool = False, workspace=None):
    """Dense causal MHA over the latent expanded per head (the path for
    prompts within top-k): q bf16 [n_q, 64, 192] (128 no-rope + 64 rope
    dims), kv bf16 [n_k, 576], w_uk / w_uv bf16 [64, 128, 512], q_pos int32
    [n_q].  Returns (out [n_q, 64, 128], lse [n_q, 64] or None)."""
    n_q = q.shape[0]
    _bf16(q, "q")
    _bf16(kv, "kv")
    _bf16(w_uk, "w_uk")
    _bf16(w_uv, "w_uv")
    if tuple(q.shape[1:]) != (HEADS, 192) or kv.shape[1] != 576:
        raise ValueError("q must be [n_q, 64, 192] and kv [n_k, 576]")
    if tuple(w_uk.shape) != (HEADS, 128, 512) or tuple(w_uv.shape) != (HEADS, 128, 512):
        raise ValueError("w_uk and w_uv must be [64, 128, 512]")
    if q_pos.dtype != torch.int32 or not q_pos.is_contiguous():
        raise ValueError("q_pos must be contiguous int32")
    dev = q.device
    if out is None:
        out = torch.empty((n_q, HEADS, 128), dtype=out_dtype, device=dev)
    odt = SMA_DT_FP32 if out.dtype == torch.float32 else SMA_DT_BF16
    lse = torch.empty((n_q, HEADS), dtype=torch.float32, device=dev) if want_lse else None
    if workspace is None:
        workspace = torch.empty(max(workspace_bytes(SMA_OP_DENSE_MHA, n_q, kv.shape[0], 1), 1), dtype=torch.uint8,
                                device=dev)
    _check(lib().sma_dense_mha_prefill(_ptr(q), _ptr(kv), _ptr(w_uk), _ptr(w_uv), _ptr(q_pos), n_q, kv.shape[0],
                                       float(sm_scale), _ptr(out), odt, _ptr(lse), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), _stream(dev)))
    return out, lse


def dcp_shard_partial(rank: int, dcp_size: int, q, kv_local, idx, sm_scale: float, *, kv_scale_local=None,
                      out=None, lse=None, workspace=None):
    """One DCP rank's partial sparse MLA over the tokens of idx (global
    positions) it stores; kv_local row j is token j*dcp_size + rank.  Returns
    (out [n_q, 64, 512] fp32, lse [n_q, 64] fp32)."""
    n_q = q.shape[0]
    _bf16(q, "q")
    kdt = _keys(kv_local, kv_scale_local, "kv_local")
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be contiguous int32")
    dev = q.device
    if out is None:
        out = torch.empty((n_q, HEADS, D_V), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((n_q, HEADS), dtype=torch.float32, device=dev)
    top_k = idx.shape[1]
    if workspace is None:
        nbytes = workspace_bytes(SMA_OP_DCP_PARTIAL, n_q, kv_local.shape[0], top_k)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    _check(lib().sma_dcp_shard_partial(rank, dcp_size, _ptr(q), _ptr(kv_local), _ptr(kv_scale_local), kdt,
                                       kv_local.shape[0], _ptr(idx), n_q, top_k, float(sm_scale), _ptr(out),
                                       _ptr(lse), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                       _stream(dev)))
    return out, lse


def dcp_shard_partial_noalloc(rank: int, dcp_size: int, q, kv_local, idx, sm_scale: float, *,
                              kv_scale_local=None, out=None, lse=None):
    """dcp_shard_partial with the library's static device scratch in place of
    a workspace (no device allocation inside the call; `out` and `lse` must
    then be given by the caller for the call to allocate nothing at all)."""
    n_q = q.shape[0]
    _bf16(q, "q")
    kdt = _keys(kv_local, kv_scale_local, "kv_local")
    if idx.dtype != torch.int32 or not idx.is_contiguous():
        raise ValueError("idx must be contiguous int32")
    dev = q.device
    if out is None:
        out = torch.empty((n_q, HEADS, D_V), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((n_q, HEADS), dtype=torch.float32, device=dev)
    top_k = idx.shape[1]
    _check(lib().sma_dcp_shard_partial_noalloc(rank, dcp_size, _ptr(q), _ptr(kv_local), _ptr(kv_scale_local), kdt,
                                               kv_local.shape[0], _ptr(idx), n_q, top_k, float(sm_scale), _ptr(out),
                                               _ptr(lse), _stream(dev)))
    return out, lse


def lse_merge(parts, lses, *, out=None, out_dtype=torch.bfloat16, want_lse: bool = False):
    """Merge partial results parts [P, n_q, 64, 512] fp32 with their lses
    [P, n_q, 64] by log-sum-exp; returns (out [n_q, 64, 512], lse or None)."""
    if parts.dtype != torch.float32 or lses.dtype != torch.float32:
        raise ValueError("parts and lses must be float32")
    if not parts.is_contiguous() or not lses.is_contiguous():
        raise ValueError("parts and lses must be contiguous")
    n_part, n_q = parts.shape[0], parts.shape[1]
    dev = parts.device
    if out is None:
        out = torch.empty((n_q, HEADS, D_V), dtype=out_dtype, device=dev)
    odt = SMA_DT_FP32 if out.dtype == torch.float32 else SMA_DT_BF16
    lse = torch.empty((n_q, HEADS), dtype=torch.float32, device=dev) if want_lse else None
    _check(lib().sma_lse_merge(_ptr(parts), _ptr(lses), n_part, n_q, _ptr(out), odt, _ptr(lse), _stream(dev)))
    return out, lse
