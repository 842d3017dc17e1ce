"""CSA2 decode hot path on MI355X: thin Python binding of the C ABI in include/csa2.h.

Argument marshalling only: every step runs in the HIP kernels of libcsa2.so.
Tensors are torch tensors on the GPU (torch supplies device memory and the
current stream); the functions check dtypes, shapes and contiguity, pass raw
pointers and sizes, and raise Csa2Error on a non-zero status.  There is no
CPU fallback: if the library is missing the calls fail loudly.

The four calls are those of one CSA2 decode layer (knowledge note
"DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache Compression", mode table
in "CSA2: share cache, refresh selection only when needed"):
quantize_kv (FP4 cache write), index_full, index_reindex, sparse_attn (Reuse
mode = sparse_attn with an earlier layer's top-k buffer).
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "Csa2Error", "lib", "load", "quantize_kv", "index_full", "index_reindex", "sparse_attn",
    "workspace_bytes", "status_str", "Workspace", "D", "DI", "PAGE", "PAGE_BYTES",
    "KIDX_PAGE_BYTES", "BLOCK", "SWA", "OP_INDEX_FULL", "OP_INDEX_REINDEX", "OP_SPARSE_ATTN",
    "index_full_noalloc", "NOALLOC_SCRATCH_BYTES", "ERR_SCRATCH", "ROW_BAD_SCALE", "ROW_UNRANKED",
    "select_path",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

D, DI, PAGE, BLOCK, SWA = 512, 128, 64, 8, 128
PAGE_BYTES, KIDX_PAGE_BYTES = 18432, 8192
MX_KIDX_PAGE_BYTES = 4352  # MXFP4 indexer keys: 64 x 64 code bytes + 64 x 4 E8M0 scales
OP_INDEX_FULL, OP_INDEX_REINDEX, OP_SPARSE_ATTN = 1, 2, 3
NOALLOC_SCRATCH_BYTES = 32 << 20  # csa2_index_full_noalloc's fixed per-GPU scratch
ERR_SCRATCH = -5
ROW_BAD_SCALE = -2   # indexer output mark: an MXFP4 key of the row has a scale code outside 119..133
ROW_UNRANKED = -3    # indexer output mark under select_path(2): the candidate path declined the row

EXPORTS = (
    "csa2_quantize_kv", "csa2_index_full", "csa2_index_reindex", "csa2_sparse_attn",
    "csa2_workspace_bytes", "csa2_status_str", "csa2_abi_version", "csa2_time_kernel",
    "csa2_test_select_path", "csa2_index_full_mxfp4", "csa2_index_reindex_mxfp4",
    "csa2_rope_write_caches", "csa2_compress", "csa2_index_full_write", "csa2_index_full_mxfp4_write",
    "csa2_index_full_noalloc", "csa2_index_full_causal", "csa2_index_reindex_causal",
)

# kernel ids for csa2_time_kernel
K_QUANTIZE, K_SCORE_FULL, K_SELECT_FULL, K_SCORE_REINDEX, K_SELECT_REINDEX = 1, 2, 3, 4, 5
K_ATTN_SPLIT, K_ATTN_COMBINE, K_ROPE_WRITE, K_COMPRESS = 6, 7, 8, 9
ROPE_PAIRS = 32  # rotary channel pairs: the last 64 channels of main-KV rows and indexer keys


class Csa2Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({status_str(status)})")
        self.status = status


_lib = None


def load(path: str = LIB_PATH):
    """Load libcsa2.so and declare the C signatures."""
    global _lib
    if _lib is not None:
        return _lib
    # torch ships its own HIP runtime (soname libamdhip64.so.7); importing it
    # first makes libcsa2.so bind to that same runtime, so torch's streams,
    # events and allocations are valid in the library.
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m compressed_sparse_attention_mxfp4_amd.build`")
    L = ctypes.CDLL(path)
    P, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.csa2_quantize_kv.argtypes = [P, i64, P, P, i64, P]
    L.csa2_rope_write_caches.argtypes = [P, P, i64, P, P, i64, P, P, P, i64, P]
    L.csa2_compress.argtypes = [P, P, i64, i32, P, P]
    L.csa2_index_full.argtypes = [P, P, P, i64, P, i32, P, i32, i32, i32, i32, i32, i32, P, P, P,
                                  P, sz, P]
    L.csa2_index_reindex.argtypes = [P, P, P, i64, P, i32, P, i32, i32, i32, P, P, i32, i32, P, P,
                                     sz, P]
    L.csa2_index_full_mxfp4.argtypes = L.csa2_index_full.argtypes
    L.csa2_index_full_write.argtypes = L.csa2_index_full.argtypes[:16] + [P, i64, P, P, i64, P, sz, P]
    L.csa2_index_full_mxfp4_write.argtypes = L.csa2_index_full_write.argtypes
    L.csa2_index_reindex_mxfp4.argtypes = L.csa2_index_reindex.argtypes
    L.csa2_index_full_noalloc.argtypes = L.csa2_index_full.argtypes[:16] + [P]
    L.csa2_index_full_causal.argtypes = L.csa2_index_full.argtypes[:7] + [P] + L.csa2_index_full.argtypes[7:]
    L.csa2_index_reindex_causal.argtypes = L.csa2_index_reindex.argtypes[:7] + [P] + L.csa2_index_reindex.argtypes[7:]
    L.csa2_sparse_attn.argtypes = [P, ctypes.c_float, P, i64, P, i32, P, P, i32, P, i32, i32, i32,
                                   P, P, P, sz, P]
    L.csa2_workspace_bytes.argtypes = [ctypes.c_int, i32, i32, i32, i32, i32]
    L.csa2_workspace_bytes.restype = sz
    L.csa2_status_str.argtypes = [ctypes.c_int]
    L.csa2_status_str.restype = ctypes.c_char_p
    L.csa2_abi_version.restype = ctypes.c_int
    L.csa2_time_kernel.argtypes = [ctypes.c_int, P, P]
    L.csa2_time_kernel.restype = ctypes.c_int
    L.csa2_test_select_path.argtypes = [ctypes.c_int]
    L.csa2_test_select_path.restype = ctypes.c_int
    for fn in ("csa2_quantize_kv", "csa2_index_full", "csa2_index_reindex", "csa2_sparse_attn",
               "csa2_index_full_mxfp4", "csa2_index_reindex_mxfp4", "csa2_rope_write_caches",
               "csa2_compress", "csa2_index_full_write", "csa2_index_full_mxfp4_write",
               "csa2_index_full_noalloc", "csa2_index_full_causal", "csa2_index_reindex_causal"):
        getattr(L, fn).restype = ctypes.c_int
    _lib = L
    return L


def lib():
    return load()


def status_str(status: int) -> str:
    return lib().csa2_status_str(int(status)).decode()


def select_path(mode: int) -> None:
    """Test aid: 0 default, 1 whole lists only, 2 candidate segments only."""
    _check("csa2_test_select_path", lib().csa2_test_select_path(int(mode)))


def workspace_bytes(op: int, B: int, T: int, heads: int, max_n_entries: int = 0, topk: int = 0) -> int:
    return int(lib().csa2_workspace_bytes(op, B, T, heads, max_n_entries, topk))


# ---------------------------------------------------------------- marshalling helpers
def _torch():
    import torch
    return torch


def _ptr(t, dtype, name, shape=None, ndim=None):
    torch = _torch()
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if shape is not None:
        for i, s in enumerate(shape):
            if s is not None and t.shape[i] != s:
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, status):
    if status != 0:
        raise Csa2Error(fn, status)


class Workspace:
    """A reusable device byte buffer, grown on demand (caller-owned scratch)."""

    def __init__(self, device="cuda"):
        self.device = device
        self.buf = None

    def get(self, nbytes: int):
        torch = _torch()
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.buf


_default_ws = {}


def _ws(ws, nbytes):
    if ws is None:
        torch = _torch()
        dev = torch.cuda.current_device()
        ws = _default_ws.setdefault(dev, Workspace(f"cuda:{dev}"))
    return ws.get(nbytes)


# ---------------------------------------------------------------- the four calls
def quantize_kv(kv_bf16, dst_slot, kv_pool, stream=None):
    """FP4 main-KV cache write: kv_bf16 [R,512] bf16, dst_slot [R] int64, kv_pool [P,18432] uint8."""
    torch = _torch()
    R = kv_bf16.shape[0]
    a = _ptr(kv_bf16, torch.bfloat16, "kv_bf16", (R, D), 2)
    s = _ptr(dst_slot, torch.int64, "dst_slot", (R,), 1)
    p = _ptr(kv_pool, torch.uint8, "kv_pool", (None, PAGE_BYTES), 2)
    _check("csa2_quantize_kv", lib().csa2_quantize_kv(a, R, s, p, kv_pool.shape[0], _stream(stream)))
    return kv_pool


def rope_write_caches(kv_bf16, kidx_bf16, pos, rope_cs, dst_slot, kv_pool, kidx_pool, stream=None):
    """Fused RoPE + cache writes: kv_bf16 [R,512] and kidx_bf16 [R,128] bf16 (pre-RoPE),
    pos [R] int64, rope_cs [max_pos,32,2] float32 (cos, sin), dst_slot [R] int64,
    kv_pool [P,18432] uint8 and kidx_pool [P,64,128] uint8 (written in place)."""
    torch = _torch()
    R = kv_bf16.shape[0]
    a = _ptr(kv_bf16, torch.bfloat16, "kv_bf16", (R, D), 2)
    k = _ptr(kidx_bf16, torch.bfloat16, "kidx_bf16", (R, DI), 2)
    p = _ptr(pos, torch.int64, "pos", (R,), 1)
    c = _ptr(rope_cs, torch.float32, "rope_cs", (None, ROPE_PAIRS, 2), 3)
    s = _ptr(dst_slot, torch.int64, "dst_slot", (R,), 1)
    kv = _ptr(kv_pool, torch.uint8, "kv_pool", (None, PAGE_BYTES), 2)
    ki = _ptr(kidx_pool, torch.uint8, "kidx_pool", (kv_pool.shape[0], PAGE, DI), 3)
    _check("csa2_rope_write_caches",
           lib().csa2_rope_write_caches(a, k, R, p, c, rope_cs.shape[0], s, kv, ki, kv_pool.shape[0],
                                        _stream(stream)))
    return kv_pool, kidx_pool


def compress(c_bf16, z_bf16, m, out=None, stream=None):
    """Sequence compressor: c_bf16, z_bf16 [R,512] bf16 -> entries [R // m, 512] bf16
    (a softmax over each group's m positions of Z weighs C, per channel)."""
    torch = _torch()
    R = c_bf16.shape[0]
    if out is None:
        out = torch.empty((R // max(int(m), 1), D), dtype=torch.bfloat16, device=c_bf16.device)
    a = _ptr(c_bf16, torch.bfloat16, "c_bf16", (R, D), 2)
    b = _ptr(z_bf16, torch.bfloat16, "z_bf16", (R, D), 2)
    o = _ptr(out, torch.bfloat16, "out", (R // max(int(m), 1), D), 2)
    _check("csa2_compress", lib().csa2_compress(a, b, R, int(m), o, _stream(stream)))
    return out


def _kidx_arg(kidx_pool, mxfp4):
    torch = _torch()
    if mxfp4:
        return _ptr(kidx_pool, torch.uint8, "kidx_pool", (None, MX_KIDX_PAGE_BYTES), 2)
    return _ptr(kidx_pool, torch.uint8, "kidx_pool", (None, PAGE, DI), 3)


def index_full(q_idx, w, kidx_pool, page_table, n_entries, max_n_entries, topk, pool_blocks=2048,
               out_topk=None, out_pool=None, out_pool_n=None, ws=None, stream=None, mxfp4=False,
               write=None, n_visible=None):
    """Full-mode indexer.  q_idx [B,T,HI,128] uint8 (E4M3), w [B,T,HI] float32,
    kidx_pool [P,64,128] uint8 E4M3 keys (or, with mxfp4=True, [P,4352] uint8 in
    the MXFP4 page layout), page_table [B,max_pages] int32, n_entries [B] int32.
    write=(kv_bf16 [R,512] bf16, dst_slot [R] int64, kv_pool [P',18432] uint8): the
    step's FP4 cache write done in the same launches.
    n_visible [B,T] int32: per-token causal visible counts (csa2_index_full_causal)."""
    torch = _torch()
    B, T, HI, _ = q_idx.shape
    dev = q_idx.device
    if out_topk is None:
        out_topk = torch.empty((B, T, topk), dtype=torch.int32, device=dev)
    if out_pool is None:
        out_pool = torch.empty((B, T, pool_blocks), dtype=torch.int32, device=dev)
    if out_pool_n is None:
        out_pool_n = torch.empty((B, T), dtype=torch.int32, device=dev)
    nb = workspace_bytes(OP_INDEX_FULL, B, T, HI, max_n_entries, topk)
    buf = _ws(ws, nb)
    args = (
        _ptr(q_idx, torch.uint8, "q_idx", (B, T, HI, DI), 4), _ptr(w, torch.float32, "w", (B, T, HI), 3),
        _kidx_arg(kidx_pool, mxfp4), kidx_pool.shape[0],
        _ptr(page_table, torch.int32, "page_table", (B, None), 2), page_table.shape[1],
        _ptr(n_entries, torch.int32, "n_entries", (B,), 1), int(max_n_entries), B, T, HI, int(topk),
        int(pool_blocks), _ptr(out_topk, torch.int32, "out_topk", (B, T, topk), 3),
        _ptr(out_pool, torch.int32, "out_pool", (B, T, pool_blocks), 3),
        _ptr(out_pool_n, torch.int32, "out_pool_n", (B, T), 2))
    tail = (ctypes.c_void_p(buf.data_ptr()), buf.numel(), _stream(stream))
    if n_visible is not None:
        if write is not None or mxfp4:
            raise ValueError("n_visible goes with E4M3 keys and no fused cache write")
        nv = _ptr(n_visible, torch.int32, "n_visible", (B, T), 2)
        name = "csa2_index_full_causal"
        st = lib().csa2_index_full_causal(*args[:7], nv, *args[7:], *tail)
    elif write is not None:
        kv_bf16, dst_slot, kv_pool = write
        R = kv_bf16.shape[0]
        wargs = (_ptr(kv_bf16, torch.bfloat16, "kv_bf16", (R, D), 2), R,
                 _ptr(dst_slot, torch.int64, "dst_slot", (R,), 1),
                 _ptr(kv_pool, torch.uint8, "kv_pool", (None, PAGE_BYTES), 2), kv_pool.shape[0])
        name = "csa2_index_full_mxfp4_write" if mxfp4 else "csa2_index_full_write"
        st = getattr(lib(), name)(*args, *wargs, *tail)
    else:
        name = "csa2_index_full_mxfp4" if mxfp4 else "csa2_index_full"
        st = getattr(lib(), name)(*args, *tail)
    _check(name, st)
    return out_topk, out_pool, out_pool_n


def index_full_noalloc(q_idx, w, kidx_pool, page_table, n_entries, max_n_entries, topk, pool_blocks=2048,
                       out_topk=None, out_pool=None, out_pool_n=None, stream=None):
    """index_full through csa2_index_full_noalloc: no workspace argument, the library's fixed
    per-GPU scratch instead (E4M3 keys)."""
    torch = _torch()
    B, T, HI, _ = q_idx.shape
    dev = q_idx.device
    if out_topk is None:
        out_topk = torch.empty((B, T, topk), dtype=torch.int32, device=dev)
    if out_pool is None:
        out_pool = torch.empty((B, T, pool_blocks), dtype=torch.int32, device=dev)
    if out_pool_n is None:
        out_pool_n = torch.empty((B, T), dtype=torch.int32, device=dev)
    st = lib().csa2_index_full_noalloc(
        _ptr(q_idx, torch.uint8, "q_idx", (B, T, HI, DI), 4), _ptr(w, torch.float32, "w", (B, T, HI), 3),
        _kidx_arg(kidx_pool, False), kidx_pool.shape[0],
        _ptr(page_table, torch.int32, "page_table", (B, None), 2), page_table.shape[1],
        _ptr(n_entries, torch.int32, "n_entries", (B,), 1), int(max_n_entries), B, T, HI, int(topk),
        int(pool_blocks), _ptr(out_topk, torch.int32, "out_topk", (B, T, topk), 3),
        _ptr(out_pool, torch.int32, "out_pool", (B, T, pool_blocks), 3),
        _ptr(out_pool_n, torch.int32, "out_pool_n", (B, T), 2), _stream(stream))
    _check("csa2_index_full_noalloc", st)
    return out_topk, out_pool, out_pool_n


def index_reindex(q_idx, w, kidx_pool, page_table, n_entries, pool, pool_n, topk, out_topk=None,
                  ws=None, stream=None, mxfp4=False, n_visible=None):
    """Reindex-mode indexer over the pool written by index_full (keys as for index_full);
    n_visible [B,T] int32: per-token causal visible counts (csa2_index_reindex_causal)."""
    torch = _torch()
    B, T, HI, _ = q_idx.shape
    P = pool.shape[2]
    if out_topk is None:
        out_topk = torch.empty((B, T, topk), dtype=torch.int32, device=q_idx.device)
    nb = workspace_bytes(OP_INDEX_REINDEX, B, T, HI, 0, topk)
    buf = _ws(ws, nb)
    head = (_ptr(q_idx, torch.uint8, "q_idx", (B, T, HI, DI), 4), _ptr(w, torch.float32, "w", (B, T, HI), 3),
            _kidx_arg(kidx_pool, mxfp4), kidx_pool.shape[0],
            _ptr(page_table, torch.int32, "page_table", (B, None), 2), page_table.shape[1],
            _ptr(n_entries, torch.int32, "n_entries", (B,), 1))
    if n_visible is not None:
        if mxfp4:
            raise ValueError("n_visible goes with E4M3 keys")
        name = "csa2_index_reindex_causal"
        head = head + (_ptr(n_visible, torch.int32, "n_visible", (B, T), 2),)
    else:
        name = "csa2_index_reindex_mxfp4" if mxfp4 else "csa2_index_reindex"
    st = getattr(lib(), name)(
        *head, B, T, HI,
        _ptr(pool, torch.int32, "pool", (B, T, P), 3), _ptr(pool_n, torch.int32, "pool_n", (B, T), 2),
        P, int(topk), _ptr(out_topk, torch.int32, "out_topk", (B, T, topk), 3),
        ctypes.c_void_p(buf.data_ptr()), buf.numel(), _stream(stream))
    _check(name, st)
    return out_topk


def sparse_attn(q, sm_scale, kv_pool, page_table, n_entries, topk_idx, swa, out=None, out_lse=None,
                ws=None, stream=None):
    """Sparse attention: q [B,T,H,512] bf16, topk_idx [B,T,k] int32, swa [B,127+T,512] uint8 (E4M3)."""
    torch = _torch()
    B, T, H, _ = q.shape
    k = topk_idx.shape[2]
    if out is None:
        out = torch.empty((B, T, H, D), dtype=torch.float32, device=q.device)
    nb = workspace_bytes(OP_SPARSE_ATTN, B, T, H, 0, k)
    buf = _ws(ws, nb)
    st = lib().csa2_sparse_attn(
        _ptr(q, torch.bfloat16, "q", (B, T, H, D), 4), float(sm_scale),
        _ptr(kv_pool, torch.uint8, "kv_pool", (None, PAGE_BYTES), 2), kv_pool.shape[0],
        _ptr(page_table, torch.int32, "page_table", (B, None), 2), page_table.shape[1],
        _ptr(n_entries, torch.int32, "n_entries", (B,), 1),
        _ptr(topk_idx, torch.int32, "topk_idx", (B, T, k), 3), k,
        _ptr(swa, torch.uint8, "swa", (B, SWA - 1 + T, D), 3), B, T, H,
        _ptr(out, torch.float32, "out", (B, T, H, D), 4),
        _ptr(out_lse, torch.float32, "out_lse", (B, T, H), 3) if out_lse is not None else None,
        ctypes.c_void_p(buf.data_ptr()), buf.numel(), _stream(stream))
    _check("csa2_sparse_attn", st)
    return out
