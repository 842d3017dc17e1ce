"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re

import pytest

import compressed_sparse_attention_mxfp4_amd as csa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
X = ctypes.c_void_p(0x1000)   # a non-null address; these calls fail before touching it


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(csa2.LIB_PATH):
        from compressed_sparse_attention_mxfp4_amd import build
        build.build()
    return csa2.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(csa2_[a-z_0-9]+)\s*\(", text, re.M)))


def test_header_declares_the_four_calls():
    names = declared_functions()
    for fn in ("csa2_quantize_kv", "csa2_index_full", "csa2_index_reindex", "csa2_sparse_attn",
               "csa2_workspace_bytes", "csa2_status_str", "csa2_abi_version"):
        assert fn in names


def test_library_exports_every_declared_symbol(L):
    for fn in declared_functions():
        assert hasattr(L, fn), fn
    assert set(csa2.EXPORTS) <= set(declared_functions())


def test_status_strings_and_version(L):
    assert csa2.status_str(0) == "ok"
    assert "workspace" in csa2.status_str(WORKSPACE)
    assert csa2.status_str(12345) == "unknown status"
    assert L.csa2_abi_version() == 108
    assert "scratch" in csa2.status_str(csa2.ERR_SCRATCH)


def test_select_path_test_aid(L):
    assert L.csa2_test_select_path(3) == INVALID
    assert L.csa2_test_select_path(-1) == INVALID
    for mode in (1, 2, 0):
        assert L.csa2_test_select_path(mode) == 0


def test_workspace_sizes(L):
    full = csa2.workspace_bytes(csa2.OP_INDEX_FULL, 4, 1, 64, 262144, 2048)
    assert full >= 4 * 262144 * 4 + 4 * 32768 * 4
    assert csa2.workspace_bytes(csa2.OP_INDEX_REINDEX, 8, 1, 64, 0, 2048) >= 8 * 16384 * 4
    # attention: a small batch splits each row list (fp32 partials of 16 heads x 512 per split);
    # a large batch keeps one split per (b, t, head tile) and needs no partials
    attn = csa2.workspace_bytes(csa2.OP_SPARSE_ATTN, 4, 1, 64, 0, 2048)
    assert attn >= 4 * 4 * 2 * 16 * 512 * 4
    assert csa2.workspace_bytes(csa2.OP_SPARSE_ATTN, 256, 1, 64, 0, 2048) <= 4096
    assert csa2.workspace_bytes(99, 1, 1, 1, 1, 1) == 0
    assert csa2.workspace_bytes(csa2.OP_INDEX_FULL, 0, 1, 64, 100, 8) == 0


def _full(L, q=X, w=X, k=X, n_pages=1, pt=X, max_pages=1, ne=X, max_n=64, B=1, T=1, HI=4, topk=8,
          pool_blocks=16, ot=X, op=X, opn=X, ws=X, ws_bytes=1 << 30):
    return L.csa2_index_full(q, w, k, n_pages, pt, max_pages, ne, max_n, B, T, HI, topk, pool_blocks,
                             ot, op, opn, ws, ws_bytes, None)


def test_index_full_argument_errors(L):
    assert _full(L, q=None) == INVALID
    assert _full(L, ot=None) == INVALID
    assert _full(L, B=0) == INVALID
    assert _full(L, topk=0) == INVALID
    assert _full(L, topk=2049, pool_blocks=2048) == INVALID
    assert _full(L, pool_blocks=4096) == INVALID
    assert _full(L, HI=6) == UNSUPPORTED
    assert _full(L, HI=68) == UNSUPPORTED
    assert _full(L, T=257) == UNSUPPORTED
    assert _full(L, B=300, T=256) == UNSUPPORTED           # B * T above 65535
    assert _full(L, topk=32, pool_blocks=16) == UNSUPPORTED
    assert _full(L, max_n=262145) == UNSUPPORTED
    assert _full(L, max_n=0) == INVALID
    assert _full(L, ws=None) == WORKSPACE
    assert _full(L, ws_bytes=16) == WORKSPACE


def test_causal_calls_need_counts(L):
    full = L.csa2_index_full_causal(X, X, X, 1, X, 1, X, None, 64, 1, 1, 4, 8, 16, X, X, X, X, 1 << 30, None)
    assert full == INVALID
    re_ = L.csa2_index_reindex_causal(X, X, X, 1, X, 1, X, None, 1, 1, 4, X, X, 16, 8, X, X, 1 << 30, None)
    assert re_ == INVALID
    assert L.csa2_index_full_causal(X, X, X, 1, X, 1, X, X, 64, 1, 257, 4, 8, 16, X, X, X, X, 1 << 30,
                                    None) == UNSUPPORTED


def test_index_full_noalloc_argument_errors(L):
    """The no-allocation call checks as csa2_index_full, then refuses what its fixed scratch cannot hold,
    all before anything is launched."""
    def call(q=X, max_n=64, B=1, T=1, HI=4, topk=8, pool_blocks=16, ot=X):
        return L.csa2_index_full_noalloc(q, X, X, 1, X, 1, X, max_n, B, T, HI, topk, pool_blocks, ot, X, X, None)
    assert call(q=None) == INVALID
    assert call(ot=None) == INVALID
    assert call(B=0) == INVALID
    assert call(max_n=0) == INVALID
    assert call(HI=6) == UNSUPPORTED
    assert call(max_n=262145) == UNSUPPORTED
    need = lambda B, T: csa2.workspace_bytes(csa2.OP_INDEX_FULL, B, T, 64, 262144, 2048)
    assert need(4, 1) <= csa2.NOALLOC_SCRATCH_BYTES            # the 1M-context batch of 4 fits
    assert need(32, 2) > csa2.NOALLOC_SCRATCH_BYTES
    assert call(max_n=262144, B=32, T=2, HI=64, topk=2048, pool_blocks=2048) == csa2.ERR_SCRATCH


def _reindex(L, q=X, pool=X, P=16, topk=8, HI=4, T=1, ws=X, ws_bytes=1 << 30, n_pages=1):
    return L.csa2_index_reindex(q, X, X, n_pages, X, 1, X, 1, T, HI, pool, X, P, topk, X, ws, ws_bytes, None)


def test_index_reindex_argument_errors(L):
    assert _reindex(L, q=None) == INVALID
    assert _reindex(L, pool=None) == INVALID
    assert _reindex(L, topk=17) == UNSUPPORTED
    assert _reindex(L, HI=10) == UNSUPPORTED
    assert _reindex(L, ws_bytes=0) == WORKSPACE
    assert _reindex(L, n_pages=(2**31 - 1) // 64 + 1) == UNSUPPORTED


def test_mxfp4_index_argument_errors(L):
    """The MXFP4-key calls share the checks of the E4M3-key ones."""
    full = lambda **kw: _full(L, **kw)
    saved = L.csa2_index_full
    try:
        L.csa2_index_full = L.csa2_index_full_mxfp4
        assert full(q=None) == INVALID
        assert full(HI=6) == UNSUPPORTED
        assert full(max_n=262145) == UNSUPPORTED
        assert full(ws=None) == WORKSPACE
    finally:
        L.csa2_index_full = saved
    r = lambda q=X, pool=X, topk=8, HI=4: L.csa2_index_reindex_mxfp4(q, X, X, 1, X, 1, X, 1, 1, HI, pool, X, 16,
                                                                     topk, X, X, 1 << 30, None)
    assert r(q=None) == INVALID
    assert r(pool=None) == INVALID
    assert r(topk=17) == UNSUPPORTED
    assert r(HI=10) == UNSUPPORTED


def _attn(L, q=X, sm=1.0, topk=8, B=1, T=1, H=16, out=X, ws=X, ws_bytes=1 << 30):
    return L.csa2_sparse_attn(q, sm, X, 1, X, 1, X, X, topk, X, B, T, H, out, None, ws, ws_bytes, None)


def test_sparse_attn_argument_errors(L):
    assert _attn(L, q=None) == INVALID
    assert _attn(L, out=None) == INVALID
    assert _attn(L, topk=0) == INVALID
    assert _attn(L, topk=4096) == INVALID
    assert _attn(L, H=48) == UNSUPPORTED
    assert _attn(L, T=257) == UNSUPPORTED
    assert _attn(L, sm=0.0) == INVALID
    assert _attn(L, sm=float("nan")) == INVALID
    assert _attn(L, ws=None) == WORKSPACE


def test_quantize_argument_errors(L):
    assert L.csa2_quantize_kv(None, 4, X, X, 1, None) == INVALID
    assert L.csa2_quantize_kv(X, -1, X, X, 1, None) == INVALID
    assert L.csa2_quantize_kv(X, 0, X, X, 1, None) == OK      # nothing to do, nothing launched


def test_rope_write_argument_errors(L):
    def call(kv=X, ki=X, rows=4, pos=X, cs=X, max_pos=100, slot=X, kvp=X, kip=X, n_pages=1):
        return L.csa2_rope_write_caches(kv, ki, rows, pos, cs, max_pos, slot, kvp, kip, n_pages, None)
    assert call(kv=None) == INVALID
    assert call(kip=None) == INVALID
    assert call(cs=None) == INVALID
    assert call(rows=-1) == INVALID
    assert call(max_pos=-1) == INVALID
    assert call(n_pages=-1) == INVALID
    assert call(cs=ctypes.c_void_p(0x1004)) == INVALID       # the angle table must be 16-byte aligned
    assert call(kv=ctypes.c_void_p(0x1008)) == INVALID       # main-KV rows must be 16-byte aligned
    assert call(ki=ctypes.c_void_p(0x1004)) == INVALID       # indexer keys must be 8-byte aligned
    assert call(max_pos=1 << 40) == UNSUPPORTED
    assert call(rows=0, kv=None, cs=None) == OK               # nothing to do, nothing launched


def test_compress_argument_errors(L):
    assert L.csa2_compress(X, X, -1, 4, X, None) == INVALID
    assert L.csa2_compress(X, X, 8, 0, X, None) == INVALID
    assert L.csa2_compress(X, X, 8, 3, X, None) == UNSUPPORTED
    assert L.csa2_compress(X, X, 8, 16, X, None) == UNSUPPORTED
    assert L.csa2_compress(None, X, 8, 4, X, None) == INVALID
    assert L.csa2_compress(X, X, 8, 4, ctypes.c_void_p(0x1008), None) == INVALID   # misaligned output
    assert L.csa2_compress(None, None, 3, 4, None, None) == OK       # no complete group, nothing launched


def test_index_full_write_argument_errors(L):
    def call(kv=X, rows=4, slot=X, pool=X, kv_pages=1, B=1):
        return L.csa2_index_full_write(X, X, X, 1, X, 1, X, 64, B, 1, 4, 8, 16, X, X, X,
                                       kv, rows, slot, pool, kv_pages, X, 1 << 30, None)
    assert call(rows=-1) == INVALID
    assert call(kv_pages=-1) == INVALID
    assert call(kv=None) == INVALID
    assert call(pool=None) == INVALID
    assert call(kv=ctypes.c_void_p(0x1008)) == INVALID            # rows must be 16-byte aligned
    assert call(rows=1025) == UNSUPPORTED
    assert call(rows=0, kv=None, slot=None, pool=None, B=0) == INVALID   # then the indexer's own checks


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(ValueError):
        csa2._ptr(torch.zeros(4), torch.float32, "x")
