"""Seeded synthetic workloads for the CSA2 decode path.

Inputs only: random draws, rounding of those draws to the storage types the
caches hold (bf16 main-KV rows before the FP4 cache write, OCP FP8 E4M3 for the
indexer keys and queries and the sliding window, done with torch's own casts),
page tables and slot lists.  None of the method's arithmetic lives here; both
the oracle tests and the HIP path draw their inputs from this module.

The five workloads follow the decode configurations the path is measured on:
a small Full layer (8K context, batch 1), a Full -> Reindex -> Reuse group at
128K context and batch 8, the 1M-token Full layer at batch 4, the 1M-row FP4
cache write, and the 20-layer decoder schedule over ragged 32K..1M contexts;
a sixth is a 256-token prefill chunk at the end of a 1M-token sequence.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

D = 512
DI = 128
PAGE = 64
SWA = 128


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator()
    g.manual_seed(int(seed))
    return g


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    """float tensor -> bf16 bit patterns (uint16), round-to-nearest-even (torch cast)."""
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def fp8_bits(x: torch.Tensor) -> np.ndarray:
    """float tensor -> OCP E4M3 codes (uint8) via torch's float8_e4m3fn cast.

    Values are drawn well inside +-448, where the cast is round-to-nearest-even."""
    return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def normal(shape, seed: int, std: float = 1.0) -> torch.Tensor:
    return torch.randn(*shape, generator=_gen(seed), dtype=torch.float32) * std


def kv_rows(n: int, seed: int, outlier_frac: float = 0.0, outlier_sigma: float = 8.0,
            channel_log10_range: tuple | None = None) -> np.ndarray:
    """Main-KV source rows (bf16 bits, [n, 512]).

    N(0,1) draws; with ``outlier_frac`` each element is independently replaced by
    +-outlier_sigma with that probability; with ``channel_log10_range`` every
    channel is multiplied by 10**U(lo, hi)."""
    g = _gen(seed)
    x = torch.randn(n, D, generator=g, dtype=torch.float32)
    if outlier_frac > 0:
        hit = torch.rand(n, D, generator=g) < outlier_frac
        sign = torch.where(torch.rand(n, D, generator=g) < 0.5, -1.0, 1.0)
        x = torch.where(hit, sign * outlier_sigma, x)
    if channel_log10_range is not None:
        lo, hi = channel_log10_range
        c = 10.0 ** (lo + (hi - lo) * torch.rand(D, generator=g, dtype=torch.float64))
        x = x * c.to(torch.float32)
    return bf16_bits(x)


def fp8_normal(shape, seed: int, std: float = 1.0) -> np.ndarray:
    return fp8_bits(normal(shape, seed, std))


def mxfp4_key_pool(n_pages: int, seed: int, scale_codes=(126,)) -> np.ndarray:
    """Random indexer-key pool in the MXFP4 page layout (uint8 [n_pages, 4352]):
    E2M1 magnitude codes drawn with the frequencies that |x| / 0.5 rounds to
    for x ~ N(0, 1) (so that, at the default scale 2^-1, the keys have the
    spread of N(0, 1) keys), random signs, and E8M0 scale codes drawn from
    `scale_codes`.  Pure random draws: no quantization happens here."""
    rng = np.random.default_rng(seed)
    mag_p = np.array([0.10, 0.19, 0.17, 0.15, 0.18, 0.13, 0.07, 0.01])
    nib = rng.choice(8, size=(n_pages, PAGE, DI), p=mag_p).astype(np.uint8)
    nib |= (rng.random((n_pages, PAGE, DI)) < 0.5).astype(np.uint8) << 3
    codes = (nib[:, :, 0::2] | (nib[:, :, 1::2] << 4)).reshape(n_pages, PAGE * DI // 2)
    scales = rng.choice(np.asarray(scale_codes, np.uint8), size=(n_pages, PAGE * 4)).astype(np.uint8)
    return np.ascontiguousarray(np.concatenate([codes, scales], axis=1))


def rope_table(max_pos: int, base: float = 10000.0) -> np.ndarray:
    """Rotary angle table float32 [max_pos, 32, 2] = (cos, sin) of pos * base^(-i/32),
    computed in binary64 and rounded once (an input: the caller chooses the angles)."""
    i = np.arange(32, dtype=np.float64)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * base ** (-i / 32.0)[None, :]
    return np.ascontiguousarray(np.stack([np.cos(ang), np.sin(ang)], axis=2).astype(np.float32))


@dataclass
class Paging:
    """Logical -> physical page mapping shared by the main-KV and indexer-key pools."""
    page_table: np.ndarray      # int32 [B, max_pages], -1 where unused
    n_entries: np.ndarray       # int32 [B]
    n_pages: int

    def slots(self, b: int) -> np.ndarray:
        """Cache slot (page * 64 + offset) of every logical entry of sequence b."""
        n = int(self.n_entries[b])
        j = np.arange(n, dtype=np.int64)
        return self.page_table[b, j // PAGE].astype(np.int64) * PAGE + j % PAGE

    def all_slots(self) -> np.ndarray:
        return np.concatenate([self.slots(b) for b in range(len(self.n_entries))])


def paging(n_entries, seed: int | None, extra_pages: int = 0) -> Paging:
    """Allocate ceil(n/64) pages per sequence; permute physical pages when seeded."""
    n_entries = np.asarray(n_entries, dtype=np.int32)
    need = [(int(n) + PAGE - 1) // PAGE for n in n_entries]
    total = sum(need) + extra_pages
    phys = np.arange(total, dtype=np.int32)
    if seed is not None:
        phys = torch.randperm(total, generator=_gen(seed)).numpy().astype(np.int32)
    max_pages = max(max(need), 1)
    pt = np.full((len(n_entries), max_pages), -1, np.int32)
    k = 0
    for b, m in enumerate(need):
        pt[b, :m] = phys[k:k + m]
        k += m
    return Paging(pt, n_entries, total)


@dataclass
class Layer:
    """Per-layer query-side inputs (each CSA2 mode computes its own query and window)."""
    mode: str                   # "full" | "reindex" | "reuse"
    q_idx: np.ndarray | None    # uint8 [B,T,HI,128] E4M3
    w: np.ndarray | None        # float32 [B,T,HI]
    q: np.ndarray               # uint16 [B,T,H,512] bf16
    swa: np.ndarray             # uint8 [B,127+T,512] E4M3


def layer_inputs(mode: str, B: int, T: int, HI: int, H: int, seed: int,
                 q_std: float = 1.0) -> Layer:
    s = 1000 * int(seed)
    if mode in ("full", "reindex"):
        q_idx = fp8_normal((B, T, HI, DI), s + 1)
        w = normal((B, T, HI), s + 2, 1.0 / math.sqrt(HI)).numpy()
    else:
        q_idx, w = None, None
    q = bf16_bits(normal((B, T, H, D), s + 3, q_std))
    swa = fp8_normal((B, SWA - 1 + T, D), s + 4)
    return Layer(mode, q_idx, w, q, swa)


@dataclass
class Workload:
    name: str
    B: int
    T: int
    H: int
    HI: int
    topk: int
    pool_blocks: int
    sm_scale: float
    n_entries: np.ndarray
    paging: Paging
    kidx_pool: np.ndarray       # uint8 [n_pages, 64, 128]
    kv_source: np.ndarray       # uint16 [sum n_entries, 512] in (b, j) order
    layers: list = field(default_factory=list)

    @property
    def max_n(self) -> int:
        return int(self.n_entries.max())


def _shared_cache(B, n_entries, seed, page_seed, outlier_frac=0.0):
    pg = paging(n_entries, page_seed)
    total = int(np.sum(n_entries))
    keys = fp8_normal((total, DI), 1000 * seed + 11)
    kidx = np.zeros((pg.n_pages, PAGE, DI), np.uint8)
    slots = pg.all_slots()
    kidx.reshape(-1, DI)[slots] = keys
    kv = kv_rows(total, 1000 * seed + 12, outlier_frac=outlier_frac)
    return pg, kidx, kv


def workload(name: str) -> Workload:
    """Named workloads (see module docstring)."""
    if name == "full_8k_b1":
        B, T, HI, H, k = 1, 1, 4, 16, 256
        n = np.array([8192 // 4], np.int32)
        pg, kidx, kv = _shared_cache(B, n, 0, None)
        L = layer_inputs("full", B, T, HI, H, 0, q_std=1.0 / math.sqrt(D))
        return Workload(name, B, T, H, HI, k, 2048, 1.0, n, pg, kidx, kv, [L])
    if name == "group_128k_b8":
        B, T, HI, H, k = 8, 1, 64, 64, 2048
        n = np.full(B, 131072 // 4, np.int32)
        pg, kidx, kv = _shared_cache(B, n, 0, 7)
        layers = [layer_inputs(m, B, T, HI, H, s) for s, m in enumerate(("full", "reindex", "reuse"))]
        return Workload(name, B, T, H, HI, k, 2048, 1.0 / math.sqrt(D), n, pg, kidx, kv, layers)
    if name == "full_1m_b4":
        B, T, HI, H, k = 4, 1, 64, 64, 2048
        n = np.full(B, 1048576 // 4, np.int32)
        pg, kidx, kv = _shared_cache(B, n, 0, 7, outlier_frac=0.01)
        L = layer_inputs("full", B, T, HI, H, 0)
        return Workload(name, B, T, H, HI, k, 2048, 1.0 / math.sqrt(D), n, pg, kidx, kv, [L])
    if name == "schedule_20l_b32":
        B, T, HI, H, k = 32, 2, 64, 64, 2048
        u = torch.rand(B, generator=_gen(20), dtype=torch.float64).numpy()
        ctx = np.round(np.exp(np.log(32768) + u * (np.log(1048576) - np.log(32768))))
        n = (ctx // 4).astype(np.int32)
        pg, kidx, kv = _shared_cache(B, n, 20, 21)
        layers = []
        for li in range(20, 40):
            mode = "full" if li == 20 else ("reindex" if li in (24, 28, 32, 36) else "reuse")
            layers.append(layer_inputs(mode, B, T, HI, H, li))
        return Workload(name, B, T, H, HI, k, 2048, 1.0 / math.sqrt(D), n, pg, kidx, kv, layers)
    if name == "prefill_256t_1m":
        # one prefill chunk of 256 query tokens at the end of a 1M-token sequence (4:1): a Full and
        # a Reindex layer of the decoder run over the chunk, each token seeing its causal prefix
        B, T, HI, H, k = 1, 256, 64, 64, 2048
        n = np.array([1048576 // 4], np.int32)
        pg, kidx, kv = _shared_cache(B, n, 30, 31)
        layers = [layer_inputs(m, B, T, HI, H, 30 + i) for i, m in enumerate(("full", "reindex"))]
        return Workload(name, B, T, H, HI, k, 2048, 1.0 / math.sqrt(D), n, pg, kidx, kv, layers)
    raise KeyError(name)


def cache_write_rows(R: int = 1048576, seed: int = 0):
    """FP4 cache-write workload: R bf16 rows with per-channel log-uniform
    [0.01, 100] scales, written page by page into a pool whose logical pages
    map to a seeded permutation of physical pages."""
    x = kv_rows(R, seed, channel_log10_range=(-2.0, 2.0))
    n_pages = (R + PAGE - 1) // PAGE
    perm = torch.randperm(n_pages, generator=_gen(seed + 1)).numpy().astype(np.int64)
    j = np.arange(R, dtype=np.int64)
    slots = perm[j // PAGE] * PAGE + j % PAGE
    return x, slots, n_pages


def kidx_rows(n: int, seed: int, channel_log10_range=(-3.0, 2.5)) -> np.ndarray:
    """Indexer-key source rows (bf16 bits, [n, 128]): N(0,1) draws times a
    per-channel 10**U(lo, hi), so that the E4M3 write meets subnormal codes
    and saturation at 448 as well as the normal range."""
    g = _gen(seed)
    x = torch.randn(n, DI, generator=g, dtype=torch.float32)
    lo, hi = channel_log10_range
    c = 10.0 ** (lo + (hi - lo) * torch.rand(DI, generator=g, dtype=torch.float64))
    return bf16_bits(x * c.to(torch.float32))


def rope_write_rows(R: int = 1048576, seed: int = 0):
    """Fused RoPE + cache-write workload: the cache-write rows and pages of
    ``cache_write_rows``, indexer-key rows from ``kidx_rows``, row j at
    position j of an R-position angle table."""
    x, slots, n_pages = cache_write_rows(R, seed)
    ki = kidx_rows(R, seed + 2)
    pos = np.arange(R, dtype=np.int64)
    return x, ki, pos, rope_table(R), slots, n_pages


def prefill_counts(n_entries, T: int, ratio: int = 4, seed: int | None = None) -> np.ndarray:
    """Per-token visible entries [B, T] (int32) of a prefill chunk whose T query tokens are the
    last T source positions of each sequence: token t of sequence b sits at position
    p = ratio * n_b + ratio - T + t and sees the floor((p + 1) / ratio) entries complete before it
    (clipped to [0, n_b]).  With ``seed``, a quarter of the tokens instead get a random count in
    [0, n_b + 16] (ragged per-token visibility, including none and more than the sequence holds)."""
    n = np.asarray(n_entries, np.int64)
    t = np.arange(T, dtype=np.int64)
    p = ratio * n[:, None] + ratio - T + t[None, :]
    out = np.clip((p + 1) // ratio, 0, n[:, None])
    if seed is not None:
        g = _gen(seed)
        hit = (torch.rand(out.shape, generator=g) < 0.25).numpy()
        rnd = (torch.rand(out.shape, generator=g, dtype=torch.float64).numpy() * (n[:, None] + 17)).astype(np.int64)
        out = np.where(hit, rnd, out)
    return out.astype(np.int32)


def random_topk(B: int, T: int, k: int, n_entries, seed: int, frac_valid: float = 1.0) -> np.ndarray:
    """Seeded index sets for attention-only tests: distinct ascending positions < n_b,
    the first ``frac_valid`` of the k slots valid, the rest -1."""
    g = _gen(seed)
    out = np.full((B, T, k), -1, np.int32)
    for b in range(B):
        n = int(n_entries[b])
        m = min(n, int(round(k * frac_valid)))
        for t in range(T):
            sel = torch.randperm(n, generator=g)[:m].numpy()
            out[b, t, :m] = np.sort(sel).astype(np.int32)
    return out
