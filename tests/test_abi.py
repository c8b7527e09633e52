"""The C-ABI library loads, exports every symbol include/sma.h declares, and
rejects bad arguments on the host before touching a device (no GPU)."""
import ctypes
import os
import re

import pytest

import sparse_mla_attention_index_amd as sma
from sparse_mla_attention_index_amd import _lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "sma.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(sma_[a-z0-9_]+)\s*\(", txt)))


def test_header_and_binding_agree():
    assert _declared() == sorted(_lib.SIGNATURES)


def test_library_exports_every_symbol():
    L = sma.lib()
    for name in _declared():
        assert getattr(L, name) is not None
    assert sma.version() >> 16 == 1
    assert L.sma_build_flags() == 0


def test_debug_library_exports_every_symbol_and_says_so():
    """The debug build has the same entry points (same ABI version) and
    reports its range checks in sma_build_flags; its host-side validation is
    the release build's."""
    D = _lib.load(_lib.DEBUG_LIB_PATH)
    for name in _declared():
        assert getattr(D, name) is not None
    assert D.sma_version() == sma.lib().sma_version()
    assert D.sma_build_flags() == _lib.SMA_BUILD_DEBUG_CHECKS
    with _lib.debug_library():
        assert _lib.build_flags() == _lib.SMA_BUILD_DEBUG_CHECKS
        assert D.sma_topk_select(None, 10, None, 4, 10, 0, None, None, 0, None) == -1
        assert "top_k" in _lib.last_error()
    assert _lib.build_flags() == 0


def test_workspace_sizes():
    # prefill: idx list + one 64-row score block (256-byte aligned pieces)
    assert sma.workspace_bytes(_lib.SMA_OP_PREFILL, 65536, 65536, 2048) == 65536 * 2048 * 4 + 64 * 65536 * 4
    # rows longer than 65,536 scores: the 64-row block also holds the split
    # top-k's buffers (per row a threshold, and per 16,384-score chunk a count
    # and a list of up to 4,096 (position, score) pairs), each 256-aligned
    def split_topk(n_q, n_k, k):
        nch = -(-n_k // 16384)
        al = lambda b: -(-b // 256) * 256
        return al(n_q * 4) + al(n_q * nch * 4) + al(n_q * nch * 4096 * 8)
    assert sma.workspace_bytes(_lib.SMA_OP_PCP_SHARE, 16384, 131072, 2048) == \
        16384 * 4 + 16384 * 2048 * 4 + 64 * 131072 * 4 + split_topk(64, 131072, 2048)
    assert sma.workspace_bytes(_lib.SMA_OP_TOPK, 10, 10, 5) == 0
    assert sma.workspace_bytes(_lib.SMA_OP_TOPK, 10, 65536, 2048) == 0
    assert sma.workspace_bytes(_lib.SMA_OP_TOPK, 64, 1 << 20, 2048) == split_topk(64, 1 << 20, 2048)
    assert sma.workspace_bytes(_lib.SMA_OP_PREFILL, 10, 100, 5) == 256 + 4096   # 200 B and 4000 B, 256-aligned
    assert sma.workspace_bytes(99, 10, 10, 5) == 0
    # attention partials for small batches: 64 queries on 256 CUs take 8 slices of
    # 64*512 + 2*64 floats each (no device here: the library assumes 256 CUs)
    assert sma.workspace_bytes(_lib.SMA_OP_SPARSE_MLA, 64, 1 << 20, 2048) == 64 * 8 * (64 * 512 + 128) * 4
    assert sma.workspace_bytes(_lib.SMA_OP_SPARSE_MLA, 65536, 65536, 2048) == 0


P = ctypes.c_void_p
FAKE = P(4096)   # never dereferenced: every call below fails validation first


@pytest.mark.parametrize("args,code,msg", [
    (dict(h=7), -2, "h_idx"),
    (dict(d=96), -2, "d_idx"),
    (dict(k=None), -1, "k_idx is NULL"),
    (dict(kdt=1), -1, "k_scale"),
    (dict(ld=5), -1, "ld_scores"),
    (dict(nq=-1), -1, "n_q"),
    (dict(nk=0), -1, "n_k"),
    (dict(wstride=3), -1, "w_stride"),
])
def test_index_scores_validation(args, code, msg):
    a = dict(h=64, d=128, k=FAKE, kdt=0, ld=10, nq=1, nk=10, wstride=64)
    a.update(args)
    r = sma.lib().sma_index_scores(FAKE, FAKE, a["wstride"], a["k"], None, a["kdt"], FAKE, a["nq"], a["nk"],
                                   a["h"], a["d"], FAKE, a["ld"], None)
    assert r == code and msg in sma.last_error()


@pytest.mark.parametrize("topk,ld,code", [(0, 10, -1), (2049, 10, -1), (5, 9, -1)])
def test_topk_validation(topk, ld, code):
    assert sma.lib().sma_topk_select(FAKE, ld, FAKE, 1, 10, topk, FAKE, None, 0, None) == code


@pytest.mark.parametrize("kvdt,scale,odt,topk,msg", [
    (1, None, 0, 8, "kv_scale"), (0, FAKE, 0, 8, "kv_scale"), (0, None, 1, 8, "out_dtype"),
    (0, None, 0, 0, "top_k"), (5, None, 0, 8, "kv_dtype"), (3, FAKE, 0, 8, "kv_scale")])
def test_mla_validation(kvdt, scale, odt, topk, msg):
    r = sma.lib().sma_sparse_mla_prefill(FAKE, FAKE, scale, kvdt, 100, FAKE, 1, topk, 0.1, FAKE, odt, None,
                                         None, 0, None)
    assert r == -1 and msg in sma.last_error()


def test_prefill_workspace_check():
    r = sma.lib().sma_prefill(FAKE, FAKE, 64, FAKE, None, 0, FAKE, FAKE, None, 0, FAKE, 16, 1000, 64, 128, 64,
                              0.1, FAKE, 0, None, None, FAKE, 100, None)
    assert r == -3 and "workspace" in sma.last_error()


@pytest.mark.parametrize("rank,P_,L,msg", [(8, 8, 1024, "rank"), (-1, 8, 1024, "rank"), (0, 8, 1000, "L_total"),
                                           (0, 0, 1024, "pcp_size")])
def test_pcp_validation(rank, P_, L, msg):
    r = sma.lib().sma_pcp_rank_share(rank, P_, L, FAKE, FAKE, 64, FAKE, None, 0, FAKE, FAKE, None, 0, 64, 128,
                                     2048, 0.1, FAKE, 0, None, None, FAKE, 1 << 40, None)
    assert r == -1 and msg in sma.last_error()


def test_c_client_built_and_rejects_bad_usage(tmp_path):
    """The plain C client of the ABI (tests/c_client) links against
    libsma.so and the HIP runtime, and reports usage and file errors with
    exit status 2 before any GPU call (its GPU run is test_gpu_c_client)."""
    import os
    import subprocess
    exe = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "tests", "c_client",
                       "prefill_client")
    assert os.path.exists(exe)
    assert subprocess.run([exe], capture_output=True, timeout=60).returncode == 2
    r = subprocess.run([exe, str(tmp_path)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "meta.txt" in r.stderr
    (tmp_path / "meta.txt").write_text("4 8 8 64 2 0.1\n")
    r = subprocess.run([exe, str(tmp_path)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "q_idx.bin" in r.stderr


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "libsma.so"))
    with pytest.raises(ImportError):
        _lib.lib()


@pytest.mark.parametrize("rank,P,msg", [(3, 3, "rank"), (-1, 3, "rank"), (0, 0, "dcp_size")])
def test_dcp_validation(rank, P, msg):
    r = sma.lib().sma_dcp_shard_partial(rank, P, FAKE, FAKE, None, 0, 100, FAKE, 1, 8, 0.1, FAKE, FAKE, FAKE,
                                        1 << 20, None)
    assert r == -1 and msg in sma.last_error()


def test_dcp_workspace_check():
    r = sma.lib().sma_dcp_shard_partial(0, 2, FAKE, FAKE, None, 0, 100, FAKE, 4, 8, 0.1, FAKE, FAKE, FAKE, 64,
                                        None)
    assert r == -3 and "workspace" in sma.last_error()
    # the local index list (256-byte aligned), then an FP8 batch's row slices
    assert sma.workspace_bytes(_lib.SMA_OP_DCP_PARTIAL, 4, 100, 8) >= 256
    assert sma.workspace_bytes(_lib.SMA_OP_DCP_PARTIAL, 65536, 65536, 2048) == 65536 * 2048 * 4


@pytest.mark.parametrize("n_part,odt,msg", [(0, 0, "n_part"), (65, 0, "n_part"), (2, 7, "out_dtype")])
def test_lse_merge_validation(n_part, odt, msg):
    r = sma.lib().sma_lse_merge(FAKE, FAKE, n_part, 3, FAKE, odt, None, None)
    assert r == -1 and msg in sma.last_error()


@pytest.mark.parametrize("n,d,code,msg", [(10, 96, -2, "d = 96"), (-1, 128, -1, "n_rows"), (10, 128, -1, "NULL")])
def test_quantize_validation(n, d, code, msg):
    r = sma.lib().sma_quantize_fp8_rows(FAKE, n, d, None if msg == "NULL" else FAKE, FAKE, None)
    assert r == code and msg in sma.last_error()


@pytest.mark.parametrize("args,code,msg", [
    (dict(h=32), -2, "64 x 128"),
    (dict(d=64), -2, "64 x 128"),
    (dict(qs=None), -1, "q_scale"),
    (dict(ks=None), -1, "k_scale"),
    (dict(ld=5), -1, "ld_scores"),
])
def test_index_scores_fp8_validation(args, code, msg):
    a = dict(h=64, d=128, qs=FAKE, ks=FAKE, ld=10)
    a.update(args)
    r = sma.lib().sma_index_scores_fp8(FAKE, a["qs"], FAKE, 64, FAKE, a["ks"], FAKE, 1, 10, a["h"], a["d"], FAKE,
                                       a["ld"], None)
    assert r == code and msg in sma.last_error()


def test_prefill_fp8_indexer_workspace_check():
    r = sma.lib().sma_prefill_fp8_indexer(FAKE, FAKE, FAKE, 64, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, 16, 1000,
                                          64, 128, 64, 0.1, FAKE, 0, None, None, FAKE, 100, None)
    assert r == -3 and "workspace" in sma.last_error()


@pytest.mark.parametrize("n,heads,ld,msg", [(-1, 64, 576, "n ="), (4, 0, 576, "heads"), (4, 64, 500, "ld_out"),
                                            (4, 64, 580, "ld_out")])
def test_absorb_q_validation(n, heads, ld, msg):
    r = sma.lib().sma_absorb_q(FAKE, FAKE, n, heads, FAKE, ld, None)
    assert r == -1 and msg in sma.last_error()


def test_project_out_validation():
    assert sma.lib().sma_project_out(FAKE, FAKE, 4, 2000, FAKE, None) == -1 and "heads" in sma.last_error()
    assert sma.lib().sma_project_out(None, FAKE, 4, 64, FAKE, None) == -1 and "NULL" in sma.last_error()


@pytest.mark.parametrize("scale", [0.0, -0.1, float("inf"), float("nan")])
def test_mla_scale_must_be_positive(scale):
    r = sma.lib().sma_sparse_mla_prefill(FAKE, FAKE, None, 0, 100, FAKE, 1, 8, scale, FAKE, 0, None, None, 0, None)
    assert r == -1 and "sm_scale" in sma.last_error()
    r = sma.lib().sma_dcp_shard_partial(0, 2, FAKE, FAKE, None, 0, 100, FAKE, 1, 8, scale, FAKE, FAKE, FAKE,
                                        1 << 20, None)
    assert r == -1 and "sm_scale" in sma.last_error()


def test_dcp_noalloc_limit():
    """The no-allocation DCP partial rejects, before any launch, an index list
    larger than its static scratch (64 MiB: 16,777,216 entries)."""
    r = sma.lib().sma_dcp_shard_partial_noalloc(0, 2, FAKE, FAKE, None, 0, 100, FAKE, 8193, 2048, 0.1, FAKE, FAKE,
                                                None)
    assert r == -3 and "static scratch" in sma.last_error()
    r = sma.lib().sma_dcp_shard_partial_noalloc(2, 2, FAKE, FAKE, None, 0, 100, FAKE, 1, 8, 0.1, FAKE, FAKE, None)
    assert r == -1 and "rank" in sma.last_error()


def test_dense_mha_validation_and_workspace():
    assert sma.workspace_bytes(_lib.SMA_OP_DENSE_MHA, 10, 2048, 1) == 2048 * 64 * 256 * 2
    L = sma.lib()
    args = lambda **k: dict(dict(q=FAKE, kv=FAKE, nq=4, nk=100, scale=0.1, odt=0, ws=FAKE, wsb=100 * 32768), **k)
    for bad, code, msg in [(dict(odt=3), -1, "out_dtype"), (dict(scale=-1.0), -1, "sm_scale"),
                           (dict(nk=0), -1, "n_k"), (dict(kv=None), -1, "NULL"),
                           (dict(wsb=100 * 32768 - 1), -3, "workspace"), (dict(ws=None), -3, "workspace")]:
        a = args(**bad)
        r = L.sma_dense_mha_prefill(a["q"], a["kv"], FAKE, FAKE, FAKE, a["nq"], a["nk"], a["scale"], FAKE, a["odt"],
                                    None, a["ws"], a["wsb"], None)
        assert r == code and msg in sma.last_error(), (bad, r, sma.last_error())
