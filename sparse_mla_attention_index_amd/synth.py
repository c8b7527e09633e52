"""Seeded synthetic inputs for the sparse-MLA prefill path.

This module only draws random numbers and packs them into the storage
formats the path consumes (bf16 as uint16 bit patterns, FP8-e4m3fn codes as
uint8 with a per-token fp32 scale).  It holds none of the method's
arithmetic: no scoring, selection or attention.  Both the CPU oracle and the
GPU path read their inputs from here, so they see identical bytes.

Every tensor is cut into fixed row blocks and each block is drawn from its
own ``PCG64`` stream keyed by (seed, tensor id, block number).  Any row range
can therefore be regenerated on its own, which is how the parity tests and
the CPU baseline sample rows of the 64K and 1M-token workloads without
drawing the whole prompt.

Workloads (shapes and distributions of the long-context prefill the GLM-5.3
PCP/DCP article discusses: 2,048 selected tokens per query, 64 heads sharing
a 576-wide latent row, FP8 KV with a 4-byte per-token scale):

==  ======================================================================
1   tiny: L=512, top_k=128, indexer 8 heads x 64, integer q_I/k_I in
    [-3, 3], w = k/16; q/kv bf16 0.1*N(0,1); output fp32
2   L=16,384, top_k=2,048, indexer 64 x 128 bf16 N(0,1), w ~ U(0,1)/8,
    q/kv bf16 N(0, 0.1^2); output bf16
3   L=65,536, as 2
4   one PCP rank's share of a 131,072-token prompt (16 chunks of 8,192)
5   decode-shaped batch: 64 queries at positions in [900,000, 1,048,575]
    over FP8 latent KV [2^20, 576] and FP8 indexer keys [2^20, 128]
==  ======================================================================
"""
from __future__ import annotations

import dataclasses
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

SEED_BASE = 20261202
N_HEADS = 64          # MLA heads sharing one latent row
D_QK = 576            # latent (512) + rope (64)
D_V = 512             # value = first 512 dims of the latent row
FP8_MAX = 448.0       # largest finite e4m3fn magnitude

_TENSOR_IDS = {"q_idx": 1, "k_idx": 2, "w": 3, "q": 4, "kv": 5, "pos": 6}
_BLOCK_ELEMS = 1 << 21


@dataclasses.dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    n_keys: int            # rows of latent KV / indexer keys
    top_k: int
    h_idx: int             # indexer heads
    d_idx: int             # indexer head dim
    int_indexer: bool      # integer-valued q_I/k_I and w = k/16
    fp8: bool              # KV and indexer keys stored as FP8 + per-token scale
    out_fp32: bool
    sm_scale: float
    pcp_size: int = 0      # >0: PCP rank share workload
    n_decode: int = 0      # >0: decode-shaped batch with drawn positions

    @property
    def seed(self) -> int:
        return SEED_BASE + self.cfg


def workload(cfg: int) -> Workload:
    tau = 1.0 / float(np.sqrt(192.0))
    if cfg == 1:
        return Workload(1, "tiny-L512-k128", 512, 128, 8, 64, True, False, True, tau)
    if cfg == 2:
        return Workload(2, "prefill-L16384-k2048", 16384, 2048, 64, 128, False, False, False, tau)
    if cfg == 3:
        return Workload(3, "prefill-L65536-k2048", 65536, 2048, 64, 128, False, False, False, tau)
    if cfg == 4:
        return Workload(4, "pcp8-share-L131072-k2048", 131072, 2048, 64, 128, False, False, False, tau,
                        pcp_size=8)
    if cfg == 5:
        return Workload(5, "decode-b64-ctx1M-fp8-k2048", 1 << 20, 2048, 64, 128, False, True, False, tau,
                        n_decode=64)
    raise ValueError(f"unknown workload {cfg}")


def _rows_per_block(row_elems: int) -> int:
    r = max(1, _BLOCK_ELEMS // row_elems)
    return 1 << (r.bit_length() - 1)


def _rng(w: Workload, tensor: str, block: int) -> np.random.Generator:
    ss = np.random.SeedSequence([w.seed, _TENSOR_IDS[tensor], block])
    return np.random.Generator(np.random.PCG64(ss))


def _draw_block(w: Workload, tensor: str, block: int, rows: int, row_elems: int) -> np.ndarray:
    """fp32 draw of one block, before any storage conversion."""
    rng = _rng(w, tensor, block)
    n = rows * row_elems
    if tensor in ("q_idx", "k_idx"):
        if w.int_indexer:
            return rng.integers(-3, 4, size=n).astype(np.float32)
        return rng.standard_normal(n, dtype=np.float32)
    if tensor == "w":
        u = rng.random(n, dtype=np.float32)
        if w.int_indexer:
            return np.round(u * 16.0).astype(np.float32) / np.float32(16.0)
        return u / np.float32(8.0)
    if tensor == "q":
        return rng.standard_normal(n, dtype=np.float32) * np.float32(0.1)
    if tensor == "kv":
        x = rng.standard_normal(n, dtype=np.float32)
        return x if w.fp8 else x * np.float32(0.1)
    raise KeyError(tensor)


def _row_elems(w: Workload, tensor: str) -> int:
    return {"q_idx": w.h_idx * w.d_idx, "k_idx": w.d_idx, "w": w.h_idx,
            "q": N_HEADS * D_QK, "kv": D_QK}[tensor]


def _gen_f32_rows(w: Workload, tensor: str, start: int, stop: int, threads: int = 8) -> np.ndarray:
    row_elems = _row_elems(w, tensor)
    rpb = _rows_per_block(row_elems)
    out = np.empty((stop - start, row_elems), dtype=np.float32)
    if stop <= start:
        return out
    b0, b1 = start // rpb, (stop - 1) // rpb

    def one(b):
        blk = _draw_block(w, tensor, b, rpb, row_elems).reshape(rpb, row_elems)
        lo, hi = max(start, b * rpb), min(stop, (b + 1) * rpb)
        out[lo - start:hi - start] = blk[lo - b * rpb:hi - b * rpb]

    blocks = range(b0, b1 + 1)
    if threads > 1 and len(blocks) > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, blocks))
    else:
        for b in blocks:
            one(b)
    return out


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest-even) and return the uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def to_fp8_rows(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-row FP8-e4m3fn storage: scale = amax/448 (fp32), codes = x/scale
    rounded to nearest-even by torch's float8_e4m3fn cast."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=1)
    scale = (amax / np.float32(FP8_MAX)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = np.clip(x / safe[:, None], -FP8_MAX, FP8_MAX)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def to_fp8_ds_mla_rows(x: np.ndarray) -> np.ndarray:
    """Latent rows [n, 576] (fp32) in FlashMLA's 656-byte fp8_ds_mla storage:
    dims 0..511 as e4m3fn codes with one fp32 scale per 128 dims (amax/448,
    codes by torch's float8_e4m3fn cast), the four scales, then dims 512..575
    as bf16 (nearest-even).  -> uint8 [n, 656]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    n = x.shape[0]
    out = np.empty((n, 656), dtype=np.uint8)
    blocks = x[:, :512].reshape(n, 4, 128)
    amax = np.abs(blocks).max(axis=2)
    scale = (amax / np.float32(FP8_MAX)).astype(np.float32)                   # [n, 4]
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = np.clip(blocks / safe[:, :, None], -FP8_MAX, FP8_MAX).reshape(n, 512)
    out[:, :512] = torch.from_numpy(np.ascontiguousarray(y)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    out[:, 512:528] = np.ascontiguousarray(scale.astype("<f4")).view(np.uint8)
    out[:, 528:] = np.ascontiguousarray(to_bf16_bits(x[:, 512:]).astype("<u2")).view(np.uint8)
    return out


def latent_rows_fp8(w: Workload, start: int, stop: int, threads: int = 8) -> tuple[np.ndarray, np.ndarray]:
    """Rows [start, stop) of the workload's latent KV as per-token FP8 (codes,
    scale) quantised from the same fp32 draws its bf16 storage rounds."""
    return to_fp8_rows(_gen_f32_rows(w, "kv", start, stop, threads))


def latent_rows_fp8_ds_mla(w: Workload, start: int, stop: int, threads: int = 8) -> np.ndarray:
    """Rows [start, stop) of the workload's latent KV in fp8_ds_mla storage
    (the same fp32 draws the other storage formats quantise)."""
    return to_fp8_ds_mla_rows(_gen_f32_rows(w, "kv", start, stop, threads))


def rows(w: Workload, tensor: str, start: int, stop: int, threads: int = 8):
    """Rows [start, stop) of one input tensor in its storage format.

    q_idx -> uint16 [n, h_idx, d_idx] (bf16 bits)
    k_idx -> uint16 [n, d_idx], or (uint8 [n, d_idx], fp32 [n]) when FP8
    w     -> float32 [n, h_idx]
    q     -> uint16 [n, 64, 576]
    kv    -> uint16 [n, 576], or (uint8 [n, 576], fp32 [n]) when FP8
    """
    x = _gen_f32_rows(w, tensor, start, stop, threads)
    n = stop - start
    if tensor == "w":
        return x
    if tensor in ("k_idx", "kv") and w.fp8:
        return to_fp8_rows(x)
    bits = to_bf16_bits(x)
    if tensor == "q_idx":
        return bits.reshape(n, w.h_idx, w.d_idx)
    if tensor == "q":
        return bits.reshape(n, N_HEADS, D_QK)
    return bits


def query_positions(w: Workload, rank: int = 0) -> np.ndarray:
    """Global positions of the workload's query rows (int32).

    Prefill: 0..L-1.  PCP share: the rows of chunks ``rank`` and
    ``2*pcp_size-1-rank`` of a prompt cut into 2*pcp_size equal chunks.
    Decode: ``n_decode`` positions drawn uniformly in [900,000, n_keys-1].
    """
    if w.n_decode:
        rng = _rng(w, "pos", 0)
        return rng.integers(900_000, w.n_keys, size=w.n_decode).astype(np.int32)
    if w.pcp_size:
        nchunk = 2 * w.pcp_size
        c = w.n_keys // nchunk
        a = np.arange(rank * c, (rank + 1) * c, dtype=np.int32)
        b = np.arange((nchunk - 1 - rank) * c, (nchunk - rank) * c, dtype=np.int32)
        return np.concatenate([a, b])
    return np.arange(w.n_keys, dtype=np.int32)


def query_rows(w: Workload, tensor: str, positions: np.ndarray, threads: int = 8):
    """Per-query tensors (q_idx, w, q) for the given global positions.

    Query-side tensors are indexed by the token's global position, so a PCP
    share or a decode batch sees the same rows the full prompt would.
    """
    positions = np.asarray(positions, dtype=np.int64)
    if positions.size == 0:
        return rows(w, tensor, 0, 0)
    # contiguous runs keep generation cheap
    order = np.argsort(positions, kind="stable")
    sp = positions[order]
    cuts = np.flatnonzero(np.diff(sp) != 1) + 1
    parts = []
    for seg in np.split(np.arange(sp.size), cuts):
        a, b = int(sp[seg[0]]), int(sp[seg[-1]]) + 1
        parts.append(rows(w, tensor, a, b, threads))
    allr = np.concatenate(parts, axis=0)
    out = np.empty_like(allr)
    out[order] = allr
    return out


def random_scores(seed: int, n_rows: int, n_cols: int, kind: str) -> np.ndarray:
    """fp32 score matrices for exercising top-k selection on its own.

    kind = "normal": continuous N(0,1) values; "ints": small integers with
    many ties; "ties": a handful of distinct values; "signed_zero": values in
    {-0.0, +0.0, 1.0} to check that the two zeros are one key; "nan" / "nan_heavy":
    N(0,1) values with about 10% / 90% of entries replaced by NaNs of both
    signs and several payloads, and a few +-inf.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([SEED_BASE, 100, seed])))
    if kind == "normal":
        return rng.standard_normal((n_rows, n_cols), dtype=np.float32)
    if kind == "ints":
        return rng.integers(0, 64, size=(n_rows, n_cols)).astype(np.float32)
    if kind == "ties":
        return rng.integers(0, 3, size=(n_rows, n_cols)).astype(np.float32) * np.float32(0.5)
    if kind == "signed_zero":
        c = rng.integers(0, 3, size=(n_rows, n_cols))
        return np.where(c == 0, np.float32(-0.0), np.where(c == 1, np.float32(0.0), np.float32(1.0))).astype(np.float32)
    if kind in ("nan", "nan_heavy"):
        x = rng.standard_normal((n_rows, n_cols), dtype=np.float32)
        u = rng.random((n_rows, n_cols))
        frac = 0.1 if kind == "nan" else 0.9
        pats = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF], dtype=np.uint32).view(np.float32)
        x = np.where(u < frac, pats[rng.integers(0, 4, size=(n_rows, n_cols))], x)
        infs = np.array([np.inf, -np.inf], dtype=np.float32)
        x = np.where((u >= frac) & (u < frac + 0.002), infs[rng.integers(0, 2, size=(n_rows, n_cols))], x)
        return x.astype(np.float32)
    raise KeyError(kind)
