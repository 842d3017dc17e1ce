"""CSA2 decode-path oracle -- test infrastructure only.

A plain, slow CPU statement of the CSA2 decode hot path, used by ``tests/``,
``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg, and by
nothing else.  The per-element arithmetic lives in ``csa2_oracle.c`` (plain C,
binary64 where the result is a real number, exact where it is discrete); this
module loads it with ctypes and composes the per-call steps the way the pages
describe the modes:

* Full    -- score every visible position, keep the top-k and build the
  block-max candidate pool ("DeepSeek-V4.1-Flash: Pushing the Limits of KV
  Cache Compression", "Hierarchical Sparse Indexer", Figure 5).
* Reindex -- score only the pool's positions with the layer's own indexer
  query, keep the top-k (same page; "Inside DeepSeek V4.1 Flash",
  "Hierarchical indexing bounds later searches").
* Reuse   -- no scoring; the latest top-k indices are used as they are
  ("CSA2: share cache, refresh selection only when needed", mode table).
* Attention over the selected dequantized FP4 entries together with the
  128-token FP8 window ("Inside DeepSeek V4.1 Flash", "CSA2: reuse memory and
  reuse selection independently"; knowledge note, "FP4 main KV").

Nothing here shares code with the HIP path; pages of the caches are gathered
with plain numpy indexing.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "csa2_oracle.c")
# (CSA2_ORACLE_LIB: another build of the same source, e.g. a sanitizer build)
_LIB = os.environ.get("CSA2_ORACLE_LIB") or os.path.join(_HERE, "libcsa2_oracle.so")

D = 512            # main-KV channels
DI = 128           # indexer-key channels
PAGE = 64          # entries per page
ENTRY_CODES = 256  # bytes of E2M1 codes per entry
NGROUPS = 32       # E4M3 scales per entry
ENTRY_BYTES = ENTRY_CODES + NGROUPS  # 288
PAGE_BYTES = PAGE * ENTRY_BYTES      # 18,432
BLOCK = 8
SWA = 128

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
             "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32, u32, dbl = ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_double
        L.csa2o_e4m3_decode.restype = dbl
        L.csa2o_e4m3_decode.argtypes = [u32]
        L.csa2o_e2m1_decode.restype = dbl
        L.csa2o_e2m1_decode.argtypes = [u32]
        L.csa2o_e4m3_nearest.restype = u32
        L.csa2o_e4m3_nearest.argtypes = [dbl]
        L.csa2o_e4m3_nearest_sixth.restype = u32
        L.csa2o_e4m3_nearest_sixth.argtypes = [dbl]
        L.csa2o_e2m1_nearest.restype = u32
        L.csa2o_e2m1_nearest.argtypes = [dbl, dbl]
        L.csa2o_quantize_row.argtypes = [P, P, P]
        L.csa2o_quantize_rows.argtypes = [P, i64, P, P]
        L.csa2o_dequant_rows.argtypes = [P, P, i64, P]
        L.csa2o_quantize_kv.argtypes = [P, i64, P, P, i64]
        L.csa2o_dequant_entry.argtypes = [P, P, P]
        L.csa2o_index_scores.argtypes = [P, P, ctypes.c_int, P, i64, P]
        L.csa2o_topk.argtypes = [P, P, i64, i32, P]
        L.csa2o_pool.argtypes = [P, i64, i32, P, P]
        L.csa2o_attention.argtypes = [P, ctypes.c_int, dbl, P, i64, P, P]
        L.csa2o_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(lib().csa2o_num_threads())


# ---------------------------------------------------------------- formats
def e4m3_decode(codes) -> np.ndarray:
    """E4M3 codes (uint8 array) -> binary64 values (NaN for S.1111.111)."""
    table = np.array([lib().csa2o_e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8)]


def e2m1_decode(codes) -> np.ndarray:
    table = np.array([lib().csa2o_e2m1_decode(c) for c in range(16)], dtype=np.float64)
    return table[np.asarray(codes, dtype=np.uint8) & 0xF]


def e4m3_nearest(x: float) -> int:
    return int(lib().csa2o_e4m3_nearest(float(x)))


def e4m3_nearest_sixth(num: float) -> int:
    return int(lib().csa2o_e4m3_nearest_sixth(float(num)))


def e2m1_nearest(a: float, s: float) -> int:
    return int(lib().csa2o_e2m1_nearest(float(a), float(s)))


def bf16_to_f64(u16) -> np.ndarray:
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- a1: cache write
def quantize_rows(x_bf16: np.ndarray):
    """x_bf16: uint16 [R, 512] -> (codes uint8 [R, 256], scales uint8 [R, 32])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16).reshape(-1, D)
    R = x.shape[0]
    codes = np.zeros((R, ENTRY_CODES), np.uint8)
    scales = np.zeros((R, NGROUPS), np.uint8)
    lib().csa2o_quantize_rows(_p(x), R, _p(codes), _p(scales))
    return codes, scales


def quantize_kv(x_bf16: np.ndarray, dst_slot: np.ndarray, pool: np.ndarray) -> np.ndarray:
    """Write rows into the paged pool (uint8 [n_pages, 18432]) in place."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16).reshape(-1, D)
    slot = np.ascontiguousarray(dst_slot, dtype=np.int64)
    assert pool.dtype == np.uint8 and pool.flags["C_CONTIGUOUS"]
    n_pages = pool.shape[0]
    lib().csa2o_quantize_kv(_p(x), x.shape[0], _p(slot), _p(pool), n_pages)
    return pool


# -------------------------------- fused RoPE + cache writes (next step)
# Knowledge note "FP4 main KV": the main KV is quantized after RoPE; the
# indexer keys are E4M3.  The pages give neither the rotary channels nor the
# angles.  Readings: the last 64 channels of each 512-channel main-KV row and
# of each 128-channel indexer key are rotary; channel pairs (2i, 2i + 1) of
# that slice turn by the angle of pair i at the row's position, given by the
# caller as a binary32 table cs[pos][i] = (cos, sin), i < 32.  With x, y the
# pair's bf16 values (exact in binary32):
#   x' = fl(fl(x c) - fl(y s)),  y' = fl(fl(x s) + fl(y c))
# every product and sum its own binary32 operation, then x', y' are rounded
# to bf16 (nearest, ties to even).  The rotated bf16 rows are written as by
# the cache write (main KV, FP4) and as E4M3 nearest-even codes saturating at
# 448 (indexer keys).
ROPE_PAIRS = 32
KV_ROPE_START, KIDX_ROPE_START = D - 2 * ROPE_PAIRS, DI - 2 * ROPE_PAIRS


def f32_to_bf16_rne(x: np.ndarray) -> np.ndarray:
    """binary32 -> bf16 bit patterns, nearest with ties to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def rope_rows(x_bf16: np.ndarray, pos: np.ndarray, rope_cs: np.ndarray, start: int) -> np.ndarray:
    """Rotate channels start .. start + 63 of bf16 rows [R, C] (see above)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16).copy()
    R = x.shape[0]
    cs = np.asarray(rope_cs, dtype=np.float32)[np.asarray(pos, dtype=np.int64)]   # [R, 32, 2]
    f = bf16_to_f64(x[:, start:start + 2 * ROPE_PAIRS]).astype(np.float32).reshape(R, ROPE_PAIRS, 2)
    xe, yo, c, sn = f[:, :, 0], f[:, :, 1], cs[:, :, 0], cs[:, :, 1]
    xr = np.subtract(np.multiply(xe, c, dtype=np.float32), np.multiply(yo, sn, dtype=np.float32), dtype=np.float32)
    yr = np.add(np.multiply(xe, sn, dtype=np.float32), np.multiply(yo, c, dtype=np.float32), dtype=np.float32)
    out = np.stack([xr, yr], axis=2).reshape(R, 2 * ROPE_PAIRS)
    x[:, start:start + 2 * ROPE_PAIRS] = f32_to_bf16_rne(out)
    return x


def e4m3_codes_of_bf16(x_bf16: np.ndarray) -> np.ndarray:
    """E4M3 nearest-even codes (saturating at 448) of bf16 values."""
    if not hasattr(e4m3_codes_of_bf16, "_t"):
        with np.errstate(invalid="ignore"):       # the NaN patterns' entries are never used
            vals = bf16_to_f64(np.arange(65536, dtype=np.uint32).astype(np.uint16))
        e4m3_codes_of_bf16._t = np.array([e4m3_nearest(v) for v in vals], dtype=np.uint8)
    table = e4m3_codes_of_bf16._t
    return table[np.asarray(x_bf16, dtype=np.uint16)]


def rope_write_caches(kv_bf16, kidx_bf16, pos, rope_cs, dst_slot, kv_pool, kidx_pool):
    """Fused RoPE + cache writes: main-KV rows [R, 512] into the FP4 pool
    [P, 18432], indexer keys [R, 128] into the E4M3 pool [P, 64, 128], in
    place; rows whose slot lies outside the pools or whose position lies
    outside the table are skipped."""
    pos = np.asarray(pos, dtype=np.int64)
    slot = np.asarray(dst_slot, dtype=np.int64)
    ok = (pos >= 0) & (pos < len(rope_cs)) & (slot >= 0) & (slot < kv_pool.shape[0] * PAGE)
    kv = rope_rows(np.asarray(kv_bf16)[ok], pos[ok], rope_cs, KV_ROPE_START)
    ki = rope_rows(np.asarray(kidx_bf16)[ok], pos[ok], rope_cs, KIDX_ROPE_START)
    quantize_kv(kv, slot[ok], kv_pool)
    codes = e4m3_codes_of_bf16(ki)
    s = slot[ok]
    kidx_pool[s // PAGE, s % PAGE] = codes
    return kv_pool, kidx_pool


# -------------------------------------------------- sequence compressor (next step)
# "Inside DeepSeek V4.1 Flash", deep dive "Causal Encoder-Decoder" (its symbol
# table and equation 1): global KV entries C and compression weights Z are
# both projected per source position, one main KV entry stands for m source
# positions, and CSA2 groups non-overlapping positions with no absolute
# positional term (section on CSA2 simplifying sequence compression).  The
# pages give no formula for how Z weighs C.  Reading: per channel, a softmax
# over the m positions of the group of Z, applied to C elementwise:
#   entry[g][c] = sum_i w_i[c] C[g m + i][c],
#   w_i[c] = exp(Z[g m + i][c]) / sum_j exp(Z[g m + j][c]).
# Only complete groups form entries.  Computed here in binary64 (the max is
# subtracted before exp, which leaves the weights unchanged).
def compress(c_bf16: np.ndarray, z_bf16: np.ndarray, m: int) -> np.ndarray:
    """Entries [G, 512] float64 of the first G = rows // m complete groups."""
    c = bf16_to_f64(np.asarray(c_bf16, dtype=np.uint16))
    z = bf16_to_f64(np.asarray(z_bf16, dtype=np.uint16))
    G = c.shape[0] // m
    c = c[:G * m].reshape(G, m, -1)
    z = z[:G * m].reshape(G, m, -1)
    e = np.exp(z - z.max(axis=1, keepdims=True))
    w = e / e.sum(axis=1, keepdims=True)
    return (w * c).sum(axis=1)


def compress_abs(c_bf16: np.ndarray, z_bf16: np.ndarray, m: int) -> np.ndarray:
    """sum_i w_i |C_i| per entry and channel (the scale of rounding errors)."""
    c = np.abs(bf16_to_f64(np.asarray(c_bf16, dtype=np.uint16)))
    return compress(f64_to_bf16_trunc(c), z_bf16, m)


def f64_to_bf16_trunc(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of values that are already bf16 (exact conversion)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "not a bf16 value"
    return (u >> 16).astype(np.uint16)


def dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    codes = np.ascontiguousarray(codes, dtype=np.uint8).reshape(-1, ENTRY_CODES)
    scales = np.ascontiguousarray(scales, dtype=np.uint8).reshape(-1, NGROUPS)
    out = np.zeros((codes.shape[0], D), np.float64)
    lib().csa2o_dequant_rows(_p(codes), _p(scales), codes.shape[0], _p(out))
    return out


def pool_entry(kv_pool: np.ndarray, page: int, off: int):
    """(codes, scales) of one entry of a paged main-KV pool."""
    base = kv_pool[page]
    return (base[off * ENTRY_CODES:(off + 1) * ENTRY_CODES],
            base[PAGE * ENTRY_CODES + off * NGROUPS:PAGE * ENTRY_CODES + (off + 1) * NGROUPS])


# ------------------------------------------- indexer keys in MXFP4 (next step)
# Knowledge note "DeepSeek-V4.1-Flash: Pushing the Limits of KV Cache
# Compression", "FP4 main KV" and "Reconstructing the 890-byte cache budget"
# on "Inside DeepSeek V4.1 Flash": the pages' own indexer-key format is E2M1
# elements with one E8M0 (power-of-two) scale per 32 channels, 68 B per
# 128-channel entry.  Reading: entry e of a page holds its 128 codes in 64
# bytes at e * 64 (channel 2i in the low nibble of byte i), the page's 64 x 4
# scale bytes follow at 4096 + e * 4 (byte g: channels 32g .. 32g + 31);
# 4,352 B per page.  E8M0 code s means 2^(s - 127).  Supported scales:
# 119 <= s <= 133 (2^-8 .. 2^6), a precondition: every key value is then a
# multiple of 2^-9 of magnitude <= 384, i.e. exactly an E4M3 value, and the
# score is the same exact function of the keys as for E4M3 keys.
MX_ENTRY_CODES = 64
MX_NGROUPS = 4
MX_ENTRY_BYTES = MX_ENTRY_CODES + MX_NGROUPS   # 68
MX_PAGE_BYTES = PAGE * MX_ENTRY_BYTES          # 4,352
MX_SCALE_MIN, MX_SCALE_MAX = 119, 133


def mxfp4_key_values(kidx_mx: np.ndarray) -> np.ndarray:
    """MXFP4 indexer-key pool uint8 [P, 4352] -> binary64 key values [P, 64, 128]."""
    pool = np.ascontiguousarray(kidx_mx, dtype=np.uint8).reshape(-1, MX_PAGE_BYTES)
    P = pool.shape[0]
    codes = pool[:, :PAGE * MX_ENTRY_CODES].reshape(P, PAGE, MX_ENTRY_CODES)
    nib = np.empty((P, PAGE, DI), np.uint8)
    nib[:, :, 0::2] = codes & 0xF
    nib[:, :, 1::2] = codes >> 4
    scales = pool[:, PAGE * MX_ENTRY_CODES:].reshape(P, PAGE, MX_NGROUPS)
    if np.any((scales < MX_SCALE_MIN) | (scales > MX_SCALE_MAX)):
        raise ValueError("E8M0 scale outside the supported range 2^-8 .. 2^6")
    scale = np.exp2(scales.astype(np.float64) - 127.0)                 # [P, 64, 4]
    return e2m1_decode(nib) * np.repeat(scale, DI // MX_NGROUPS, axis=2)


def mxfp4_keys_to_e4m3(kidx_mx: np.ndarray) -> np.ndarray:
    """The same keys as E4M3 codes [P, 64, 128]: an exact re-encoding under the
    scale precondition (raises if a code/scale pair has no E4M3 code)."""
    pool = np.ascontiguousarray(kidx_mx, dtype=np.uint8).reshape(-1, MX_PAGE_BYTES)
    mxfp4_key_values(pool[:1])  # format check on one page; the full check follows below
    scales = pool[:, PAGE * MX_ENTRY_CODES:].reshape(pool.shape[0], PAGE, MX_NGROUPS)
    if np.any((scales < MX_SCALE_MIN) | (scales > MX_SCALE_MAX)):
        raise ValueError("E8M0 scale outside the supported range 2^-8 .. 2^6")
    # table[s, c]: the E4M3 code whose value is exactly E2M1(c) * 2^(s - 127)
    e4 = e4m3_decode(np.arange(256))
    e2 = e2m1_decode(np.arange(16))
    table = np.zeros((256, 16), np.uint8)
    for sc in range(MX_SCALE_MIN, MX_SCALE_MAX + 1):
        for c in range(16):
            x = e2[c] * 2.0 ** (sc - 127)
            hit = [k for k in range(256) if e4[k] == x and np.signbit(e4[k]) == np.signbit(x)]
            if not hit:
                raise ValueError(f"E2M1 code {c} at scale code {sc} has no E4M3 code")
            table[sc, c] = hit[0]
    codes = pool[:, :PAGE * MX_ENTRY_CODES].reshape(pool.shape[0], PAGE, MX_ENTRY_CODES)
    nib = np.empty((pool.shape[0], PAGE, DI), np.uint8)
    nib[:, :, 0::2] = codes & 0xF
    nib[:, :, 1::2] = codes >> 4
    sc_ch = np.repeat(scales, DI // MX_NGROUPS, axis=2)
    return table[sc_ch, nib]


# ---------------------------------------------------------------- a2..a6: indexer
def index_scores(q_codes: np.ndarray, w: np.ndarray, key_codes: np.ndarray) -> np.ndarray:
    """q_codes uint8 [H,128], w float32 [H], key_codes uint8 [n,128] -> float32 [n]."""
    q = np.ascontiguousarray(q_codes, dtype=np.uint8)
    w = np.ascontiguousarray(w, dtype=np.float32)
    k = np.ascontiguousarray(key_codes, dtype=np.uint8).reshape(-1, DI)
    if q.shape[0] > 64:
        raise ValueError("the score's head sum has 64 slots: at most 64 indexer heads")
    s = np.zeros(k.shape[0], np.float32)
    lib().csa2o_index_scores(_p(q), _p(w), q.shape[0], _p(k), k.shape[0], _p(s))
    return s


def topk(s: np.ndarray, k: int, idx: np.ndarray | None = None) -> np.ndarray:
    s = np.ascontiguousarray(s, dtype=np.float32)
    out = np.zeros(k, np.int32)
    if idx is not None:
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        lib().csa2o_topk(_p(s), _p(idx), s.shape[0], k, _p(out))
    else:
        lib().csa2o_topk(_p(s), None, s.shape[0], k, _p(out))
    return out


def pool(s: np.ndarray, pool_blocks: int):
    s = np.ascontiguousarray(s, dtype=np.float32)
    out = np.zeros(pool_blocks, np.int32)
    n = ctypes.c_int32(0)
    lib().csa2o_pool(_p(s), s.shape[0], pool_blocks, _p(out), ctypes.byref(n))
    return out, int(n.value)


def gather_keys(kidx_pool: np.ndarray, page_table_row: np.ndarray, n: int) -> np.ndarray:
    """Logical indexer keys [n,128] of one sequence from the paged pool [P,64,128]."""
    j = np.arange(n)
    return kidx_pool[page_table_row[j // PAGE], j % PAGE]


def pool_positions(pool_blocks_row: np.ndarray, n_blocks: int, n: int) -> np.ndarray:
    """Positions covered by the first n_blocks pool blocks, ascending."""
    pos = []
    for b in pool_blocks_row[:n_blocks]:
        pos.extend(range(8 * int(b), min(8 * int(b) + 8, n)))
    return np.array(pos, dtype=np.int32)


def visible_count(n_entries, n_visible, b: int, t: int) -> int:
    """Entries token t of sequence b sees: all n_entries[b], or with per-token causal
    counts the first min(n_entries[b], n_visible[b, t]) ("Inside DeepSeek V4.1 Flash",
    "CED": a prefill token sees only the compressed entries complete before it)."""
    n = int(n_entries[b])
    if n_visible is not None:
        n = max(0, min(n, int(n_visible[b, t])))
    return n


def index_full(q_idx, w, kidx_pool, page_table, n_entries, topk_k, pool_blocks, n_visible=None):
    """Full mode for a batch: returns (topk [B,T,k], pool [B,T,pool_blocks], pool_n [B,T]).
    n_visible [B,T]: optional per-token causal visible counts."""
    B, T, HI, _ = q_idx.shape
    out_topk = np.zeros((B, T, topk_k), np.int32)
    out_pool = np.zeros((B, T, pool_blocks), np.int32)
    out_n = np.zeros((B, T), np.int32)
    for b in range(B):
        all_keys = gather_keys(kidx_pool, page_table[b], int(n_entries[b]))
        for t in range(T):
            keys = all_keys[:visible_count(n_entries, n_visible, b, t)]
            s = index_scores(q_idx[b, t], w[b, t], keys)
            out_topk[b, t] = topk(s, topk_k)
            out_pool[b, t], out_n[b, t] = pool(s, pool_blocks)
    return out_topk, out_pool, out_n


def index_full_mxfp4(q_idx, w, kidx_mx, page_table, n_entries, topk_k, pool_blocks):
    """Full mode over MXFP4 indexer keys (same outputs as index_full)."""
    return index_full(q_idx, w, mxfp4_keys_to_e4m3(kidx_mx), page_table, n_entries, topk_k, pool_blocks)


def index_reindex_mxfp4(q_idx, w, kidx_mx, page_table, n_entries, pool_, pool_n, topk_k):
    """Reindex mode over MXFP4 indexer keys (same output as index_reindex)."""
    return index_reindex(q_idx, w, mxfp4_keys_to_e4m3(kidx_mx), page_table, n_entries, pool_, pool_n, topk_k)


def index_reindex(q_idx, w, kidx_pool, page_table, n_entries, pool_, pool_n, topk_k, n_visible=None):
    """Reindex mode: score only the pool's positions; returns topk [B,T,k].
    n_visible [B,T]: optional per-token causal visible counts (pool blocks are clipped to them)."""
    B, T, HI, _ = q_idx.shape
    out = np.zeros((B, T, topk_k), np.int32)
    for b in range(B):
        for t in range(T):
            n = visible_count(n_entries, n_visible, b, t)
            pos = pool_positions(pool_[b, t], int(pool_n[b, t]), n)
            pt = page_table[b]
            keys = kidx_pool[pt[pos // PAGE], pos % PAGE] if len(pos) else np.zeros((0, DI), np.uint8)
            s = index_scores(q_idx[b, t], w[b, t], keys)
            out[b, t] = topk(s, topk_k, pos)
    return out


# ---------------------------------------------------------------- a7: attention
def attention(q: np.ndarray, sm_scale: float, rows: np.ndarray):
    """q float64 [H,512], rows float64 [nr,512] -> (out [H,512], lse [H])."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    rows = np.ascontiguousarray(rows, dtype=np.float64).reshape(-1, D)
    H = q.shape[0]
    out = np.zeros((H, D), np.float64)
    lse = np.zeros(H, np.float64)
    lib().csa2o_attention(_p(q), H, float(sm_scale), _p(rows), rows.shape[0], _p(out), _p(lse))
    return out, lse


def selected_rows(kv_pool, page_table_row, idx_row):
    """Dequantized main-KV rows of the valid (>= 0) selected positions."""
    sel = [int(j) for j in idx_row if j >= 0]
    if not sel:
        return np.zeros((0, D), np.float64)
    codes = np.stack([pool_entry(kv_pool, int(page_table_row[j // PAGE]), j % PAGE)[0] for j in sel])
    scales = np.stack([pool_entry(kv_pool, int(page_table_row[j // PAGE]), j % PAGE)[1] for j in sel])
    return dequant(codes, scales)


def sparse_attn_from_rows(q_bf16_bt, sm_scale, sel_rows_bf16, swa_rows):
    """Attention of one (b, t) given the bf16 source rows of its selected entries.

    The oracle writes those rows to FP4 with its own cache-write statement,
    dequantizes them, and attends over them plus the 128 FP8 window rows."""
    if len(sel_rows_bf16):
        codes, scales = quantize_rows(sel_rows_bf16)
        rows = dequant(codes, scales)
    else:
        rows = np.zeros((0, D), np.float64)
    allrows = np.concatenate([rows, e4m3_decode(swa_rows)], axis=0)
    return attention(bf16_to_f64(q_bf16_bt), sm_scale, allrows)


def sparse_attn(q_bf16, sm_scale, kv_pool, page_table, topk_idx, swa, batches=None, tokens=None):
    """Attention for each (b, t): softmax over the selected entries plus SWA rows t..t+127.

    q_bf16 uint16 [B,T,H,512]; kv_pool uint8 [P,18432]; topk_idx int32 [B,T,k];
    swa uint8 [B,127+T,512] (E4M3).  Returns (out float64 [B,T,H,512], lse [B,T,H]);
    only the (b, t) pairs listed in ``batches``/``tokens`` are computed (others NaN).
    """
    B, T, H, _ = q_bf16.shape
    out = np.full((B, T, H, D), np.nan)
    lse = np.full((B, T, H), np.nan)
    for b in (range(B) if batches is None else batches):
        for t in (range(T) if tokens is None else tokens):
            rows = selected_rows(kv_pool, page_table[b], topk_idx[b, t])
            win = e4m3_decode(swa[b, t:t + SWA])
            allrows = np.concatenate([rows, win], axis=0)
            out[b, t], lse[b, t] = attention(bf16_to_f64(q_bf16[b, t]), sm_scale, allrows)
    return out, lse
