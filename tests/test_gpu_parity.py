"""GPU parity: the HIP path (through the C ABI) against the oracle.

FP4 codes, scales, top-k and pool index sets must match bit for bit; attention
outputs within max-abs 2e-3 of the binary64 oracle given the same indices.
Inputs come from the seeded generators only; the oracle never sees a value
the HIP path produced except where noted (index sets fed to both sides after
they have been shown equal).
"""
import math
import sys

import numpy as np
import pytest
import torch

import compressed_sparse_attention_mxfp4_amd as csa2
from compressed_sparse_attention_mxfp4_amd import synth

pytestmark = pytest.mark.gpu

ATOL = 2e-3


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    csa2.load()
    yield
    torch.cuda.synchronize()


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bf16_dev(u16):
    return dev(u16.view(np.int16), torch.bfloat16) if u16.dtype == np.uint16 else dev(u16)


# ------------------------------------------------------------------ a1
def gpu_quantize(x_u16, slots, n_pages, fill=0xAA):
    pool = torch.full((n_pages, csa2.PAGE_BYTES), fill, dtype=torch.uint8, device="cuda")
    csa2.quantize_kv(bf16_dev(x_u16), dev(slots.astype(np.int64)), pool)
    return host(pool)


def special_rows():
    """Hand-picked groups: every E2M1 tie, scale ties, subnormal and zero scales, saturation, -0."""
    vals = [
        [6.0, -3.0, 1.0, 0.5, 0.25, 0.75, -0.0, 0.0, 2.5, 5.0, 4.0, 1.25, 1.75, 3.5, 0.30078125, 0.125],
        [7.0, 1.0] + [0.0] * 14,
        [6.375, -6.375] + [0.0] * 14,
        [0.01171875, 0.0029296875] + [0.0] * 14,
        [-0.005859375, 0.005859375] + [0.0] * 14,
        [3072.0, 1000.0] + [0.0] * 14,
        [-0.0] * 16,
        [1e-30, -1e-30] + [0.0] * 14,
        [60000.0, -1.0] + [0.0] * 14,
        # scale 1.125 (amax 6.75) and 1.875 (amax 11.25): every E2M1 tie times the scale
        [6.75, 0.28125, 0.84375, 1.40625, 1.96875, 2.8125, 3.9375, 5.625,
         -0.28125, -0.84375, -1.40625, -1.96875, -2.8125, -3.9375, -5.625, 0.0],
        [11.25, 0.46875, 1.40625, 2.34375, 3.28125, 4.6875, 6.5625, 9.375,
         -0.46875, -1.40625, -2.34375, -3.28125, -4.6875, -6.5625, -9.375, -0.0],
    ]
    rows = []
    for v in vals:
        row = np.tile(np.array(v, np.float32), 32)
        rows.append(row)
    return synth.bf16_bits(torch.tensor(np.stack(rows)))


def test_quantize_parity_mixed(oracle):
    say("quantize mixed 6000 rows")
    x = np.concatenate([
        synth.kv_rows(2000, 1),
        synth.kv_rows(2000, 2, outlier_frac=0.05),
        synth.kv_rows(2000, 3, channel_log10_range=(-2.0, 2.0)),
        special_rows(),
    ])
    n_pages = (len(x) + 63) // 64 + 3
    rng = np.random.default_rng(0)
    slots = rng.permutation(n_pages * 64)[:len(x)].astype(np.int64)
    slots[5] = -1
    slots[6] = n_pages * 64 + 3
    got = gpu_quantize(x, slots, n_pages)
    ref = np.full((n_pages, oracle.PAGE_BYTES), 0xAA, np.uint8)
    oracle.quantize_kv(x, slots, ref)
    assert np.array_equal(got, ref)


def test_quantize_parity_full_cache_write(oracle):
    say("quantize 1,048,576 rows, log-uniform channel scales, permuted pages")
    x, slots, n_pages = synth.cache_write_rows()
    got = gpu_quantize(x, slots, n_pages, fill=0)
    codes, scales = oracle.quantize_rows(x)
    page, off = slots // 64, slots % 64
    gc = got[:, :64 * 256].reshape(n_pages, 64, 256)[page, off]
    gs = got[:, 64 * 256:].reshape(n_pages, 64, 32)[page, off]
    assert np.array_equal(gc, codes)
    assert np.array_equal(gs, scales)


# ------------------------------------------------------------------ fused RoPE + cache writes
def gpu_rope_write(kv, ki, pos, table, slots, n_pages, fill=0xAA):
    kvp = torch.full((n_pages, csa2.PAGE_BYTES), fill, dtype=torch.uint8, device="cuda")
    kip = torch.full((n_pages, 64, 128), fill, dtype=torch.uint8, device="cuda")
    csa2.rope_write_caches(bf16_dev(kv), bf16_dev(ki), dev(pos.astype(np.int64)), dev(table),
                           dev(slots.astype(np.int64)), kvp, kip)
    return host(kvp), host(kip)


def oracle_rope_write(oracle, kv, ki, pos, table, slots, n_pages, fill=0xAA):
    kvp = np.full((n_pages, oracle.PAGE_BYTES), fill, np.uint8)
    kip = np.full((n_pages, 64, 128), fill, np.uint8)
    return oracle.rope_write_caches(kv, ki, pos, table, slots, kvp, kip)


def test_rope_write_parity_mixed(oracle):
    say("rope write 6011 rows: special groups, outliers, wide scales, skipped rows")
    kv = np.concatenate([synth.kv_rows(2000, 11), synth.kv_rows(2000, 12, outlier_frac=0.05),
                         synth.kv_rows(2000, 13, channel_log10_range=(-2.0, 2.0)), special_rows()])
    R = len(kv)
    ki = synth.kidx_rows(R, 14)
    table = synth.rope_table(4096)
    rng = np.random.default_rng(3)
    pos = rng.integers(0, len(table), R).astype(np.int64)
    n_pages = (R + 63) // 64 + 2
    slots = rng.permutation(n_pages * 64)[:R].astype(np.int64)
    slots[5], slots[6] = -1, n_pages * 64 + 3          # skipped: slot outside the pools
    pos[7], pos[8] = -1, len(table)                     # skipped: position outside the table
    got_kv, got_ki = gpu_rope_write(kv, ki, pos, table, slots, n_pages)
    ref_kv, ref_ki = oracle_rope_write(oracle, kv, ki, pos, table, slots, n_pages)
    assert np.array_equal(got_kv, ref_kv)
    assert np.array_equal(got_ki, ref_ki)


def test_rope_write_e4m3_every_finite_bf16(oracle):
    say("rope write: every finite bf16 pattern through the E4M3 key write")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = bits[(bits & 0x7F80) != 0x7F80]             # 65,024 patterns = 1016 x 64
    n = len(finite) // 64
    ki = np.zeros((n, 128), np.uint16)
    ki[:, :64] = finite.reshape(n, 64)                  # the channels that do not rotate
    ki[:, 64:] = finite.reshape(n, 64)[::-1]            # and the rotary ones, turned by angle 0
    kv = synth.kv_rows(n, 15)
    table = synth.rope_table(3)
    pos = np.zeros(n, np.int64)
    slots = np.arange(n, dtype=np.int64)
    n_pages = (n + 63) // 64
    got_kv, got_ki = gpu_rope_write(kv, ki, pos, table, slots, n_pages)
    assert np.array_equal(got_ki.reshape(-1, 128)[:n, :64].reshape(-1), oracle.e4m3_codes_of_bf16(finite))
    ref_kv, ref_ki = oracle_rope_write(oracle, kv, ki, pos, table, slots, n_pages)
    assert np.array_equal(got_ki, ref_ki)
    assert np.array_equal(got_kv, ref_kv)


def test_rope_write_parity_full(oracle):
    say("rope write 1,048,576 rows at positions 0 .. 2^20 - 1, permuted pages")
    kv, ki, pos, table, slots, n_pages = synth.rope_write_rows()
    got_kv, got_ki = gpu_rope_write(kv, ki, pos, table, slots, n_pages, fill=0)
    ref_kv, ref_ki = oracle_rope_write(oracle, kv, ki, pos, table, slots, n_pages, fill=0)
    assert np.array_equal(got_ki, ref_ki)
    assert np.array_equal(got_kv, ref_kv)


# ------------------------------------------------------------------ sequence compressor
def check_compress(oracle, c, z, m, got):
    """|got - exact| <= 2^-8 |exact| (the bf16 rounding) + (1 + 2^-8) e32, where e32 bounds the
    binary32 steps per channel: e32 = 2^-24 sum_i w_i |C_i| (2m + 4 + 2 |d_i|), d_i = Z_i - max_j Z_j.
    Per term: the exponent argument d_i log2(e) carries a relative error <= 2^-23, which scales the
    weight by at most |d_i| 2^-23; v_exp_f32 adds <= 2^-23 (1 ulp); the m - 1 adds of the positive
    weights and the m fused multiply-adds add <= (2m - 1) 2^-24 of the weighted sum; the correctly
    rounded quotient 2^-24."""
    exact = oracle.compress(c, z, m)
    groups = exact.shape[0]
    cf = oracle.bf16_to_f64(c[: groups * m]).reshape(groups, m, -1)
    zf = oracle.bf16_to_f64(z[: groups * m]).reshape(groups, m, -1)
    d = zf - zf.max(axis=1, keepdims=True)
    w = np.exp(d)
    w /= w.sum(axis=1, keepdims=True)
    e32 = 2.0 ** -24 * np.sum(w * np.abs(cf) * (2 * m + 4 + 2 * np.abs(d)), axis=1)
    g = got.astype(np.float64)
    err = np.abs(g - exact)
    bound = 2.0 ** -8 * np.abs(exact) + (1 + 2.0 ** -8) * e32
    assert g.shape == exact.shape
    assert np.all(err <= bound), float(np.max(err / np.maximum(bound, 1e-300)))
    # the share of entries equal to the bf16 nearest the exact value (the rest sit within the
    # binary32 error of a rounding boundary)
    near = oracle.f32_to_bf16_rne(exact.astype(np.float32))
    return float(np.mean(oracle.bf16_to_f64(near) == g))


@pytest.mark.parametrize("m", [1, 2, 4, 8])
def test_compress_parity(oracle, m):
    R = 8 * 301 + 5                                  # ragged: a partial trailing group for m > 1
    say(f"compress m={m} rows={R}")
    c = synth.kv_rows(R, 70 + m, channel_log10_range=(-2.0, 2.0))
    z = synth.kv_rows(R, 80 + m, outlier_frac=0.02)  # weights from near-uniform to one dominant position
    got = csa2.compress(bf16_dev(c), bf16_dev(z), m)
    g = host(got.view(torch.int16)).view(np.uint16)
    frac = check_compress(oracle, c, z, m, oracle.bf16_to_f64(g))
    say(f"compress m={m}: {frac:.4f} of entries equal to the exact value's nearest bf16")
    assert frac > 0.99


def test_compress_full_4to1(oracle):
    say("compress 4:1, 1,048,576 source rows -> 262,144 entries, sampled against the oracle")
    R = 1 << 20
    c = synth.kv_rows(R, 90)
    z = synth.kv_rows(R, 91)
    got = csa2.compress(bf16_dev(c), bf16_dev(z), 4)
    g = host(got.view(torch.int16)).view(np.uint16)
    rng = np.random.default_rng(5)
    pick = np.sort(rng.choice(R // 4, 4096, replace=False))
    rows = (pick[:, None] * 4 + np.arange(4)[None, :]).reshape(-1)
    check_compress(oracle, c[rows], z[rows], 4, oracle.bf16_to_f64(g[pick]))


def test_rope_write_and_compress_edges(oracle):
    say("rope write: one row; empty angle table (every row skipped); compress: no complete group, one group")
    kv, ki = synth.kv_rows(1, 31), synth.kidx_rows(1, 32)
    table = synth.rope_table(10)
    pos, slots = np.array([9], np.int64), np.array([70], np.int64)   # last position, page 1 offset 6
    got_kv, got_ki = gpu_rope_write(kv, ki, pos, table, slots, 2)
    ref_kv, ref_ki = oracle_rope_write(oracle, kv, ki, pos, table, slots, 2)
    assert np.array_equal(got_kv, ref_kv) and np.array_equal(got_ki, ref_ki)
    kv, ki = synth.kv_rows(5, 33), synth.kidx_rows(5, 34)
    got_kv, got_ki = gpu_rope_write(kv, ki, np.zeros(5, np.int64), np.zeros((0, 32, 2), np.float32),
                                    np.arange(5, dtype=np.int64), 1)
    assert np.all(got_kv == 0xAA) and np.all(got_ki == 0xAA)
    c, z = synth.kv_rows(8, 35), synth.kv_rows(8, 36)
    none = csa2.compress(bf16_dev(c[:3]), bf16_dev(z[:3]), 4)
    assert tuple(none.shape) == (0, 512)
    one = csa2.compress(bf16_dev(c), bf16_dev(z), 8)
    check_compress(oracle, c, z, 8, oracle.bf16_to_f64(host(one.view(torch.int16)).view(np.uint16)))


# ------------------------------------------------------------------ a2..a6
def gpu_index_full(wl, layer, topk=None, pool_blocks=None):
    topk = topk or wl.topk
    pool_blocks = pool_blocks or wl.pool_blocks
    return csa2.index_full(dev(layer.q_idx), dev(layer.w), dev(wl.kidx_pool),
                           dev(wl.paging.page_table), dev(wl.n_entries), wl.max_n, topk, pool_blocks)


def oracle_index_full(oracle, wl, layer, topk=None, pool_blocks=None):
    return oracle.index_full(layer.q_idx, layer.w, wl.kidx_pool, wl.paging.page_table, wl.n_entries,
                             topk or wl.topk, pool_blocks or wl.pool_blocks)


def assert_index_equal(got, ref):
    for g, r in zip(got, ref):
        assert np.array_equal(host(g), r)


def small_workload(n_entries, T=1, HI=8, H=16, topk=64, seed=0, key_codes=None, q_codes=None):
    pg = synth.paging(n_entries, seed=seed + 3)
    kidx = np.zeros((pg.n_pages, 64, 128), np.uint8)
    total = int(np.sum(n_entries))
    keys = synth.fp8_normal((total, 128), seed + 9) if key_codes is None else key_codes
    kidx.reshape(-1, 128)[pg.all_slots()] = keys
    L = synth.layer_inputs("full", len(n_entries), T, HI, H, seed)
    if q_codes is not None:
        L.q_idx = q_codes
    kv = synth.kv_rows(total, seed + 12)
    return synth.Workload("small", len(n_entries), T, H, HI, topk, 2048, 1 / math.sqrt(512),
                          np.asarray(n_entries, np.int32), pg, kidx, kv, [L])


def test_index_full_8k_b1(oracle):
    say("index full 8K ctx B=1 HI=4 k=256")
    wl = synth.workload("full_8k_b1")
    got = gpu_index_full(wl, wl.layers[0])
    assert_index_equal(got, oracle_index_full(oracle, wl, wl.layers[0]))


def _e4m3_value(codes):
    c = codes.astype(np.int64)
    e, m = (c >> 3) & 15, (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8 * 2.0**-6, (1 + m / 8) * 2.0 ** (e - 7))
    return np.where(c & 0x80, -mag, mag)


def _bounded_extreme_keys(rows, rng):
    """Keys at the edge of the scan's fast path (sum_c k_c^2 < 500), random signs:
    mode 0: one channel of 22, 20, 18 or 16 over subnormal and tiny channels,
            so large and tiny products meet in one accumulation;
    mode 1: 112..128 channels of 1.75 or 1.875 (sum |k| up to 240, so the
            partial sums reach 128 * 240) and the rest subnormal;
    mode 2: every channel 2.0 (sum k^2 = 512): just past the bound, left to
            the general path."""
    keys = np.zeros((rows, 128), np.uint8)
    for j in range(rows):
        mode = j % 3
        tiny = rng.integers(0, 16, 128).astype(np.uint8)
        if mode == 0:
            row = tiny
            row[rng.integers(0, 128)] = rng.choice(np.array([0x5B, 0x5A, 0x59, 0x58], np.uint8))
        elif mode == 1:
            row = rng.choice(np.array([0x3E, 0x3F], np.uint8), 128)
            n_small = rng.integers(0, 17)
            row[rng.permutation(128)[:n_small]] = tiny[:n_small] & 7
        else:
            row = np.full(128, 0x40, np.uint8)
        keys[j] = row | (rng.integers(0, 2, 128).astype(np.uint8) << 7)
    sq = (_e4m3_value(keys) ** 2).sum(axis=1)
    assert (sq[0::3] < 500).all() and (sq[1::3] < 500).all() and (sq[2::3] >= 500).all()
    return keys


@pytest.mark.parametrize("keys_kind", ["normal", "all_codes", "bounded_extreme"])
def test_index_full_scores_bitexact(oracle, keys_kind):
    """The scan's scores, bit for bit: Full mode keeps them in the first region
    of its workspace, [B][T][max_n rounded up to 8] float32 (NaN where not
    visible).  "all_codes" keys run every finite E4M3 code (general path);
    "bounded_extreme" keys and queries sit at the edge of the fast path's
    exactness bound (sum k^2 < 500, |q| < 32)."""
    n = [3000, 1000, 777]
    say(f"index full scores bit-exact n={n} T=2 HI=64 keys={keys_kind}")
    key_codes = q_codes = None
    rng = np.random.default_rng(11)
    if keys_kind == "all_codes":
        finite = np.array([c for c in range(256) if c not in (127, 255)], np.uint8)
        key_codes = rng.choice(finite, (sum(n), 128))
    if keys_kind == "bounded_extreme":
        key_codes = _bounded_extreme_keys(sum(n), rng)
        # query codes with |q| <= 30 (exponent field <= 11), many near the top
        qc = rng.integers(0, 0x5F, (len(n), 2, 64, 128)).astype(np.uint8)
        qc[..., ::3] = 0x5E  # 28
        q_codes = qc | (rng.integers(0, 2, qc.shape).astype(np.uint8) << 7)
    wl = small_workload(n, T=2, HI=64, topk=256, seed=21, key_codes=key_codes, q_codes=q_codes)
    L = wl.layers[0]
    ws = csa2.Workspace()
    csa2.index_full(dev(L.q_idx), dev(L.w), dev(wl.kidx_pool), dev(wl.paging.page_table),
                    dev(wl.n_entries), wl.max_n, wl.topk, wl.pool_blocks, ws=ws)
    stride = (wl.max_n + 7) & ~7
    s_gpu = host(ws.buf)[: len(n) * 2 * stride * 4].view(np.float32).reshape(len(n), 2, stride)
    for b, nb in enumerate(n):
        keys = oracle.gather_keys(wl.kidx_pool, wl.paging.page_table[b], nb)
        for t in range(2):
            ref = oracle.index_scores(L.q_idx[b, t], L.w[b, t], keys)
            assert np.array_equal(s_gpu[b, t, :nb].view(np.uint32), ref.view(np.uint32)), (b, t)


@pytest.mark.parametrize("T,HI,topk", [(1, 8, 64), (2, 16, 512), (4, 4, 2048), (2, 64, 2048), (3, 8, 256),
                                       (6, 16, 512)])
def test_index_full_ragged(oracle, T, HI, topk):
    n = [1, 7, 8, 9, 100, 1023, 1025, 2047, 2048, 16389, 40000]
    say(f"index full ragged n={n} T={T} HI={HI} k={topk}")
    wl = small_workload(n, T=T, HI=HI, topk=topk, seed=T * 100 + HI)
    got = gpu_index_full(wl, wl.layers[0])
    assert_index_equal(got, oracle_index_full(oracle, wl, wl.layers[0]))


@pytest.mark.parametrize("mx", [False, True])
def test_index_full_with_fused_cache_write(oracle, mx):
    say(f"index_full{'_mxfp4' if mx else ''}_write: Full indexer with the step's cache write in the same launches")
    wl = small_workload([30000, 12345], T=2, HI=32, topk=1024, seed=12)
    L = wl.layers[0]
    keys = synth.mxfp4_key_pool(wl.paging.n_pages, 14) if mx else wl.kidx_pool
    rows = synth.kv_rows(37, 13, outlier_frac=0.02)       # 37 rows: a partial last wave
    n_pages = wl.paging.n_pages
    slots = np.random.default_rng(4).permutation(n_pages * 64)[:37].astype(np.int64)
    slots[3] = -1
    kv = torch.full((n_pages, csa2.PAGE_BYTES), 0xAA, dtype=torch.uint8, device="cuda")
    tk, pl, pn = csa2.index_full(dev(L.q_idx), dev(L.w), dev(keys), dev(wl.paging.page_table),
                                 dev(wl.n_entries), wl.max_n, wl.topk, wl.pool_blocks, mxfp4=mx,
                                 write=(bf16_dev(rows), dev(slots), kv))
    if mx:
        r_tk, r_pool, r_pn = oracle.index_full_mxfp4(L.q_idx, L.w, keys, wl.paging.page_table, wl.n_entries,
                                                     wl.topk, wl.pool_blocks)
    else:
        r_tk, r_pool, r_pn = oracle_index_full(oracle, wl, L)
    assert np.array_equal(host(tk), r_tk) and np.array_equal(host(pl), r_pool) and np.array_equal(host(pn), r_pn)
    ref = np.full((n_pages, oracle.PAGE_BYTES), 0xAA, np.uint8)
    oracle.quantize_kv(rows, slots, ref)
    assert np.array_equal(host(kv), ref)


def test_empty_sequence_index_and_attention(oracle):
    """A sequence with no entries: its top-k is all -1, its pool empty, and its
    attention runs over the window rows alone."""
    n = [0, 5, 3000]
    say(f"index + attention with an empty sequence n={n} T=2 HI=8 k=64")
    wl = small_workload(n, T=2, HI=8, topk=64, seed=61)
    L = wl.layers[0]
    got = gpu_index_full(wl, L)
    ref = oracle_index_full(oracle, wl, L)
    assert_index_equal(got, ref)
    assert (ref[0][0] == -1).all() and (ref[2][0] == 0).all()
    kv_pool = torch.zeros((max(wl.paging.n_pages, 1), csa2.PAGE_BYTES), dtype=torch.uint8, device="cuda")
    csa2.quantize_kv(bf16_dev(wl.kv_source), dev(wl.paging.all_slots()), kv_pool)
    out = csa2.sparse_attn(bf16_dev(L.q), wl.sm_scale, kv_pool, dev(wl.paging.page_table), dev(wl.n_entries),
                           got[0], dev(L.swa))
    check_attention(oracle, wl, L, ref[0], host(out))


def test_index_full_ties(oracle):
    say("index full with tied scores (repeated keys)")
    n = [5000, 700]
    base = synth.fp8_normal((7, 128), 77)
    rng = np.random.default_rng(3)
    keys = base[rng.integers(0, 7, sum(n))]
    wl = small_workload(n, T=2, HI=8, topk=256, seed=5, key_codes=keys)
    got = gpu_index_full(wl, wl.layers[0])
    assert_index_equal(got, oracle_index_full(oracle, wl, wl.layers[0]))


@pytest.mark.parametrize("distinct", [1, 3, 50])
def test_index_full_max_entries_heavy_ties(oracle, distinct):
    """262,144 entries (the maximum) drawn from a few distinct keys: thousands of
    equal block maxima and scores, so both selections break ties by index over
    the whole list (distinct=1: every score equal)."""
    say(f"index full 262,144 entries from {distinct} distinct key(s)")
    n = [262144, 131075]
    base = synth.fp8_normal((distinct, 128), 70 + distinct)
    rng = np.random.default_rng(distinct)
    keys = base[rng.integers(0, distinct, sum(n))]
    wl = small_workload(n, T=1, HI=4, topk=2048, seed=11, key_codes=keys)
    got = gpu_index_full(wl, wl.layers[0])
    assert_index_equal(got, oracle_index_full(oracle, wl, wl.layers[0]))


def test_index_full_all_scores_zero(oracle):
    say("index full with zero queries: every score is +0")
    n = [262144, 9]
    wl = small_workload(n, T=2, HI=4, topk=2048, seed=12, q_codes=np.zeros((2, 2, 4, 128), np.uint8))
    got = gpu_index_full(wl, wl.layers[0])
    ref = oracle_index_full(oracle, wl, wl.layers[0])
    assert (ref[0][0, 0] == np.arange(2048)).all()  # ties go to the lowest indices
    assert_index_equal(got, ref)


def test_index_full_wide_exponent_range(oracle):
    say("index full with every finite E4M3 code (general exact path)")
    n = [3000, 999]
    rng = np.random.default_rng(4)
    finite = np.array([c for c in range(256) if c not in (127, 255)], np.uint8)
    keys = rng.choice(finite, (sum(n), 128))
    q = rng.choice(finite, (2, 1, 16, 128))
    wl = small_workload(n, T=1, HI=16, topk=128, seed=6, key_codes=keys, q_codes=q)
    got = gpu_index_full(wl, wl.layers[0])
    assert_index_equal(got, oracle_index_full(oracle, wl, wl.layers[0]))


def test_index_full_1m_b4(oracle):
    say("index full 1M ctx B=4 HI=64 k=2048 (full size)")
    wl = synth.workload("full_1m_b4")
    got = gpu_index_full(wl, wl.layers[0])
    ref = oracle_index_full(oracle, wl, wl.layers[0])
    assert_index_equal(got, ref)
    # the pool bounds: <= 2,048 blocks of 8 positions, and the top-k lies inside it
    tk, pool_, pool_n = ref
    assert (pool_n == 2048).all()
    for b in range(wl.B):
        pos = oracle.pool_positions(pool_[b, 0], int(pool_n[b, 0]), int(wl.n_entries[b]))
        assert len(pos) <= 16384 and set(tk[b, 0]) <= set(pos)


# ------------------------------------------------------------------ MXFP4 indexer keys
@pytest.mark.parametrize("scales", ["typical", "range_edges"])
def test_index_full_mxfp4_scores_bitexact(oracle, scales):
    """Full mode over MXFP4 indexer keys: the scan's scores bit for bit, and the
    top-k and pool, against the oracle.  "range_edges" draws scale codes at both
    ends of the supported range (2^-8, 2^-7, 2^5, 2^6), so large keys send
    chunks to the general path and tiny ones stay on the fast path."""
    n = [3000, 1000, 777]
    sc = (125, 126, 127) if scales == "typical" else (119, 120, 132, 133)
    say(f"index full MXFP4 keys, scores bit-exact n={n} T=2 HI=64 scales={sc}")
    wl = small_workload(n, T=2, HI=64, topk=256, seed=31)
    mx = synth.mxfp4_key_pool(wl.paging.n_pages, 41, sc)
    L = wl.layers[0]
    ws = csa2.Workspace()
    got = csa2.index_full(dev(L.q_idx), dev(L.w), dev(mx), dev(wl.paging.page_table), dev(wl.n_entries),
                          wl.max_n, wl.topk, wl.pool_blocks, ws=ws, mxfp4=True)
    stride = (wl.max_n + 7) & ~7
    s_gpu = host(ws.buf)[: len(n) * 2 * stride * 4].view(np.float32).reshape(len(n), 2, stride)
    e4 = oracle.mxfp4_keys_to_e4m3(mx)
    for b, nb in enumerate(n):
        keys = oracle.gather_keys(e4, wl.paging.page_table[b], nb)
        for t in range(2):
            ref = oracle.index_scores(L.q_idx[b, t], L.w[b, t], keys)
            assert np.array_equal(s_gpu[b, t, :nb].view(np.uint32), ref.view(np.uint32)), (b, t)
    ref = oracle.index_full_mxfp4(L.q_idx, L.w, mx, wl.paging.page_table, wl.n_entries, wl.topk,
                                  wl.pool_blocks)
    assert_index_equal(got, ref)


@pytest.mark.parametrize("T,HI,topk", [(1, 8, 64), (4, 16, 2048)])
def test_index_full_and_reindex_mxfp4_ragged(oracle, T, HI, topk):
    n = [1, 7, 9, 1025, 16389, 40000]
    say(f"index full + reindex MXFP4 keys ragged n={n} T={T} HI={HI} k={topk}")
    wl = small_workload(n, T=T, HI=HI, topk=topk, seed=T * 10 + HI)
    mx = synth.mxfp4_key_pool(wl.paging.n_pages, 43)
    L = wl.layers[0]
    other = synth.layer_inputs("full", wl.B, T, HI, 16, 44)
    args = (dev(mx), dev(wl.paging.page_table), dev(wl.n_entries))
    got = csa2.index_full(dev(L.q_idx), dev(L.w), *args, wl.max_n, topk, 2048, mxfp4=True)
    ref = oracle.index_full_mxfp4(L.q_idx, L.w, mx, wl.paging.page_table, wl.n_entries, topk, 2048)
    assert_index_equal(got, ref)
    rtk = csa2.index_reindex(dev(other.q_idx), dev(other.w), *args, got[1], got[2], topk, mxfp4=True)
    ref_rtk = oracle.index_reindex_mxfp4(other.q_idx, other.w, mx, wl.paging.page_table, wl.n_entries,
                                         ref[1], ref[2], topk)
    assert np.array_equal(host(rtk), ref_rtk)


def test_index_full_mxfp4_1m_b4(oracle):
    say("index full 1M ctx B=4 HI=64 k=2048 over MXFP4 keys (full size)")
    wl = synth.workload("full_1m_b4")
    mx = synth.mxfp4_key_pool(wl.paging.n_pages, 45)
    L = wl.layers[0]
    got = csa2.index_full(dev(L.q_idx), dev(L.w), dev(mx), dev(wl.paging.page_table), dev(wl.n_entries),
                          wl.max_n, wl.topk, wl.pool_blocks, mxfp4=True)
    ref = oracle.index_full_mxfp4(L.q_idx, L.w, mx, wl.paging.page_table, wl.n_entries, wl.topk,
                                  wl.pool_blocks)
    assert_index_equal(got, ref)


def test_index_deterministic():
    say("index full twice, identical")
    wl = small_workload([30000, 12345], T=2, HI=32, topk=1024, seed=9)
    a = [host(x) for x in gpu_index_full(wl, wl.layers[0])]
    b = [host(x) for x in gpu_index_full(wl, wl.layers[0])]
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("mode", [1, 2])
def test_index_selection_paths(oracle, mode):
    """The selections rank the union of the scan's candidate segments when they can show it
    holds the exact top-k and pool, and the whole lists otherwise.  Mode 1 ranks the whole lists
    always, mode 2 the segments only (a row they cannot rank would read ROW_UNRANKED); on random
    scores both give the oracle's Full and Reindex results on every row."""
    say(f"index full + reindex, selection path mode {mode}")
    wl = small_workload([40000, 9000, 262144], T=2, HI=16, topk=512, seed=21)
    other = synth.layer_inputs("full", wl.B, wl.T, 16, 16, 22)
    layer = wl.layers[0]
    args = (dev(wl.kidx_pool), dev(wl.paging.page_table), dev(wl.n_entries))
    ref = oracle_index_full(oracle, wl, layer)
    ref_rtk = oracle.index_reindex(other.q_idx, other.w, wl.kidx_pool, wl.paging.page_table,
                                   wl.n_entries, ref[1], ref[2], wl.topk)
    csa2.select_path(mode)
    try:
        got = csa2.index_full(dev(layer.q_idx), dev(layer.w), *args, wl.max_n, wl.topk, 2048)
        rtk = csa2.index_reindex(dev(other.q_idx), dev(other.w), *args, got[1], got[2], wl.topk)
        torch.cuda.synchronize()
    finally:
        csa2.select_path(0)
    assert_index_equal(got, ref)
    assert np.array_equal(host(rtk), ref_rtk)


def test_index_segments_decline_when_all_scores_tie(oracle):
    """One sequence of 262,144 entries whose scores are all +0: every workgroup keeps all of its
    keys, more than the selection takes from segments, so the candidate path declines the row
    (mode 2: every slot and the count read ROW_UNRANKED) and the default path ranks the whole
    lists, ties to the lowest indices, as the oracle does."""
    say("index full 262,144 equal scores: the candidate path declines, the whole lists rank")
    wl = small_workload([262144], T=1, HI=4, topk=2048, seed=13, q_codes=np.zeros((1, 1, 4, 128), np.uint8))
    ref = oracle_index_full(oracle, wl, wl.layers[0])
    csa2.select_path(2)
    try:
        declined = [host(x) for x in gpu_index_full(wl, wl.layers[0])]
    finally:
        csa2.select_path(0)
    for x in declined:
        assert (x == csa2.ROW_UNRANKED).all()
    assert_index_equal(gpu_index_full(wl, wl.layers[0]), ref)


def test_index_mxfp4_bad_scale_rows_reported(oracle):
    """MXFP4 keys whose scale code lies outside 119..133 are reported, not ranked: a (b, t) row
    whose scanned entries hold one reads ROW_BAD_SCALE in every top-k slot (Full: also every pool
    slot and the count); a bad code in an entry the row does not see changes nothing, and the
    other rows equal the oracle.  The oracle (which refuses such codes) sees the pool before the
    codes were changed: the rows compared with it do not read the changed entries."""
    n = [3000, 1000, 777]
    say(f"index full + reindex MXFP4 with out-of-range scale codes n={n}")
    wl = small_workload(n, T=2, HI=16, topk=256, seed=33)
    mx_ok = synth.mxfp4_key_pool(wl.paging.n_pages, 47)
    mx = mx_ok.copy()
    pt = wl.paging.page_table

    def set_scale(b, j, g, code):
        mx[pt[b, j // 64], 4096 + (j % 64) * 4 + g] = code

    set_scale(0, 3005, 1, 200)   # past n[0] on an allocated page: not visible
    set_scale(1, 500, 2, 118)    # below the range
    set_scale(2, 776, 0, 134)    # the last visible entry, above the range
    L = wl.layers[0]
    args = (dev(mx), dev(pt), dev(wl.n_entries))
    tk, pl, pn = csa2.index_full(dev(L.q_idx), dev(L.w), *args, wl.max_n, wl.topk, 2048, mxfp4=True)
    ref = oracle.index_full_mxfp4(L.q_idx, L.w, mx_ok, pt, wl.n_entries, wl.topk, 2048)
    tk, pl, pn = host(tk), host(pl), host(pn)
    assert np.array_equal(tk[0], ref[0][0]) and np.array_equal(pl[0], ref[1][0]) and np.array_equal(pn[0], ref[2][0])
    for b in (1, 2):
        assert (tk[b] == csa2.ROW_BAD_SCALE).all() and (pl[b] == csa2.ROW_BAD_SCALE).all()
        assert (pn[b] == csa2.ROW_BAD_SCALE).all()
    # Reindex over the oracle's pools: a row is reported when its pool holds the bad entry
    other = synth.layer_inputs("full", wl.B, 2, 16, 16, 48)
    rtk = host(csa2.index_reindex(dev(other.q_idx), dev(other.w), *args, dev(ref[1]), dev(ref[2]), wl.topk,
                                  mxfp4=True))
    ref_rtk = oracle.index_reindex_mxfp4(other.q_idx, other.w, mx_ok, pt, wl.n_entries, ref[1], ref[2], wl.topk)
    n_reported = 0
    for b in range(3):
        for t in range(2):
            blocks = set(ref[1][b, t, : ref[2][b, t]].tolist())
            bad = (b == 1 and 500 // 8 in blocks) or (b == 2 and 776 // 8 in blocks)
            if bad:
                n_reported += 1
                assert (rtk[b, t] == csa2.ROW_BAD_SCALE).all(), (b, t)
            else:
                assert np.array_equal(rtk[b, t], ref_rtk[b, t]), (b, t)
    # sequence 2 has 98 blocks, all in its pools
    assert n_reported >= 2


def test_group_128k_b8_full_reindex_reuse(oracle):
    say("group 128K ctx B=8: Full -> Reindex -> Reuse")
    wl = synth.workload("group_128k_b8")
    full, reidx, reuse = wl.layers
    tk, pool_, pool_n = gpu_index_full(wl, full)
    ref_tk, ref_pool, ref_pool_n = oracle_index_full(oracle, wl, full)
    assert np.array_equal(host(tk), ref_tk)
    assert np.array_equal(host(pool_), ref_pool)
    assert np.array_equal(host(pool_n), ref_pool_n)
    rtk = csa2.index_reindex(dev(reidx.q_idx), dev(reidx.w), dev(wl.kidx_pool), dev(wl.paging.page_table),
                             dev(wl.n_entries), pool_, pool_n, wl.topk)
    ref_rtk = oracle.index_reindex(reidx.q_idx, reidx.w, wl.kidx_pool, wl.paging.page_table,
                                   wl.n_entries, ref_pool, ref_pool_n, wl.topk)
    assert np.array_equal(host(rtk), ref_rtk)
    # Reindex stays inside the pool; Reuse takes the Reindex buffer unchanged
    for b in range(wl.B):
        pos = set(oracle.pool_positions(ref_pool[b, 0], int(ref_pool_n[b, 0]), int(wl.n_entries[b])))
        assert set(ref_rtk[b, 0]) <= pos
    kv_pool = torch.zeros((wl.paging.n_pages, csa2.PAGE_BYTES), dtype=torch.uint8, device="cuda")
    csa2.quantize_kv(bf16_dev(wl.kv_source), dev(wl.paging.all_slots()), kv_pool)
    before = host(rtk).copy()
    out = csa2.sparse_attn(bf16_dev(reuse.q), wl.sm_scale, kv_pool, dev(wl.paging.page_table),
                           dev(wl.n_entries), rtk, dev(reuse.swa))
    assert np.array_equal(host(rtk), before)
    check_attention(oracle, wl, reuse, ref_rtk, host(out), batches=[0, 3, 7])


@pytest.mark.parametrize("T,n,HI,H,topk", [(64, [20000, 3001], 64, 64, 2048), (256, [16384], 16, 16, 512)])
def test_prefill_causal_full_reindex_attention(oracle, T, n, HI, H, topk):
    """A prefill chunk of T query tokens per sequence, each token seeing only its causal share of
    the entries: Full and Reindex top-k, pools and counts bit-exact per token, attention within
    the bound on sampled tokens."""
    say(f"prefill chunk T={T} n={n} HI={HI} H={H} k={topk}: causal Full -> Reindex -> attention")
    wl = small_workload(n, T=T, HI=HI, H=H, topk=topk, seed=T)
    full = wl.layers[0]
    reidx = synth.layer_inputs("reindex", wl.B, T, HI, H, T + 1)
    n_vis = synth.prefill_counts(n, T, seed=T + 2)
    pt, ne, nv = dev(wl.paging.page_table), dev(wl.n_entries), dev(n_vis)
    tk, pl, pn = csa2.index_full(dev(full.q_idx), dev(full.w), dev(wl.kidx_pool), pt, ne, wl.max_n, topk, 2048,
                                 n_visible=nv)
    r_tk, r_pool, r_pn = oracle.index_full(full.q_idx, full.w, wl.kidx_pool, wl.paging.page_table, wl.n_entries,
                                           topk, 2048, n_visible=n_vis)
    assert np.array_equal(host(pn), r_pn)
    assert np.array_equal(host(pl), r_pool)
    assert np.array_equal(host(tk), r_tk)
    rtk = csa2.index_reindex(dev(reidx.q_idx), dev(reidx.w), dev(wl.kidx_pool), pt, ne, pl, pn, topk,
                             n_visible=nv)
    r_rtk = oracle.index_reindex(reidx.q_idx, reidx.w, wl.kidx_pool, wl.paging.page_table, wl.n_entries, r_pool,
                                 r_pn, topk, n_visible=n_vis)
    assert np.array_equal(host(rtk), r_rtk)
    out, _ = gpu_attention(wl, full, r_rtk)
    check_attention(oracle, wl, full, r_rtk, out, tokens=[0, 1, T // 2, T - 1])


def test_schedule_20l_b32_full_size(oracle):
    """The 20-layer decoder schedule at full size: batch 32, 2 query tokens, ragged contexts
    (8,342 .. 252,139 entries).  Layer 20 is Full (with the step's cache write), layers 24, 28,
    32, 36 Reindex over layer 20's pool, the rest Reuse the latest indices.  Every Full and
    Reindex top-k, pool and count is bit-exact for all 64 rows; attention is within the bound on
    sampled rows of Full, Reindex and Reuse layers; Reuse leaves the index buffers unchanged."""
    say("schedule 20 layers B=32 T=2 ragged 32K..1M: Full -> 4 x Reindex, attention per layer")
    wl = synth.workload("schedule_20l_b32")
    pt, ne = dev(wl.paging.page_table), dev(wl.n_entries)
    kidx = dev(wl.kidx_pool)
    kv_pool = torch.zeros((wl.paging.n_pages, csa2.PAGE_BYTES), dtype=torch.uint8, device="cuda")
    csa2.quantize_kv(bf16_dev(wl.kv_source), dev(wl.paging.all_slots()), kv_pool)
    by = {20 + i: L for i, L in enumerate(wl.layers)}
    L = by[20]
    tk, pl, pn = csa2.index_full(dev(L.q_idx), dev(L.w), kidx, pt, ne, wl.max_n, wl.topk, wl.pool_blocks)
    r_tk, r_pool, r_pn = oracle_index_full(oracle, wl, L)
    assert np.array_equal(host(pn), r_pn)
    assert np.array_equal(host(pl), r_pool)
    assert np.array_equal(host(tk), r_tk)
    say("schedule: Full layer 20 bit-exact on all 64 rows")
    latest = {20: (tk, r_tk)}
    for li in (24, 28, 32, 36):
        R = by[li]
        rtk = csa2.index_reindex(dev(R.q_idx), dev(R.w), kidx, pt, ne, pl, pn, wl.topk)
        r_rtk = oracle.index_reindex(R.q_idx, R.w, wl.kidx_pool, wl.paging.page_table, wl.n_entries, r_pool, r_pn,
                                     wl.topk)
        assert np.array_equal(host(rtk), r_rtk), li
        latest[li] = (rtk, r_rtk)
    say("schedule: Reindex layers 24, 28, 32, 36 bit-exact on all 64 rows")
    order = np.argsort(wl.n_entries)
    sample = sorted({int(order[0]), int(order[len(order) // 2]), int(order[-1]), 5})
    for li in (20, 21, 24, 27, 36, 39):
        src = max(x for x in latest if x <= li)
        idx, ref_idx = latest[src]
        before = host(idx).copy()
        out = csa2.sparse_attn(bf16_dev(by[li].q), wl.sm_scale, kv_pool, pt, ne, idx, dev(by[li].swa))
        assert np.array_equal(host(idx), before)
        check_attention(oracle, wl, by[li], ref_idx, host(out), batches=sample)


# ------------------------------------------------------------------ a7
def check_attention(oracle, wl, layer, idx, out, batches=None, tokens=None, lse=None):
    offs = np.concatenate([[0], np.cumsum(wl.n_entries)[:-1]])
    worst = 0.0
    for b in (range(wl.B) if batches is None else batches):
        for t in (range(wl.T) if tokens is None else tokens):
            sel = [int(j) for j in idx[b, t] if j >= 0]
            rows = wl.kv_source[offs[b] + np.array(sel, dtype=np.int64)] if sel else np.zeros((0, 512), np.uint16)
            ref, ref_lse = oracle.sparse_attn_from_rows(layer.q[b, t], wl.sm_scale, rows,
                                                        layer.swa[b, t:t + 128])
            err = np.abs(out[b, t] - ref).max()
            worst = max(worst, err)
            assert err <= ATOL, (b, t, err)
            if lse is not None:
                assert np.abs(lse[b, t] - ref_lse).max() <= 1e-3
    say(f"attention max-abs error {worst:.3g}")
    return worst


def gpu_attention(wl, layer, idx, with_lse=False):
    kv_pool = torch.zeros((wl.paging.n_pages, csa2.PAGE_BYTES), dtype=torch.uint8, device="cuda")
    csa2.quantize_kv(bf16_dev(wl.kv_source), dev(wl.paging.all_slots()), kv_pool)
    lse = torch.empty((wl.B, wl.T, wl.H), dtype=torch.float32, device="cuda") if with_lse else None
    out = csa2.sparse_attn(bf16_dev(layer.q), wl.sm_scale, kv_pool, dev(wl.paging.page_table),
                           dev(wl.n_entries), dev(idx) if isinstance(idx, np.ndarray) else idx,
                           dev(layer.swa), out_lse=lse)
    return host(out), (host(lse) if with_lse else None)


def test_attention_8k_b1(oracle):
    say("attention 8K ctx B=1 H=16 k=256 (indices from the Full layer)")
    wl = synth.workload("full_8k_b1")
    L = wl.layers[0]
    ref_tk, _, _ = oracle_index_full(oracle, wl, L)
    out, lse = gpu_attention(wl, L, ref_tk, with_lse=True)
    check_attention(oracle, wl, L, ref_tk, out, lse=lse)


# 64 heads at B*T < 8 run the head-tile kernel, at B*T >= 8 (T >= 3 here,
# three sequences) the all-heads kernel; k = 100 and 2,047 leave a sub-chunk
# holding both top-k and window rows
@pytest.mark.parametrize("H,T,k,frac", [(16, 1, 256, 1.0), (32, 2, 512, 0.7), (64, 1, 2048, 0.5),
                                        (64, 2, 2048, 1.0), (16, 4, 8, 1.0), (64, 1, 100, 0.0),
                                        (64, 3, 2048, 0.5), (64, 4, 100, 0.0), (64, 3, 2047, 1.0),
                                        (32, 32, 2048, 0.8)])
def test_attention_random_index_sets(oracle, H, T, k, frac):
    say(f"attention random sets H={H} T={T} k={k} valid={frac}")
    n = [5000, 300, 9999]
    wl = small_workload(n, T=T, H=H, topk=k, seed=H + T + k)
    L = synth.layer_inputs("reuse", wl.B, T, 0, H, 17, q_std=1.0)
    idx = synth.random_topk(wl.B, T, k, wl.n_entries, seed=k, frac_valid=frac)
    out, lse = gpu_attention(wl, L, idx, with_lse=True)
    check_attention(oracle, wl, L, idx, out, lse=lse)


@pytest.mark.parametrize("H,T", [(64, 1), (64, 8), (16, 2)])
def test_attention_query_magnitudes(oracle, H, T):
    """Queries whose heads span 2^-24 .. 2^24 in scale (bf16, some far above fp16's 65,504, some
    below its normal range): every head's fp16 operand is the bf16 query times a power of two
    (exact), so the outputs stay within the bound on both attention kernels."""
    say(f"attention with query heads scaled 2^-24 .. 2^24, H={H} T={T}")
    n = [3000, 777]
    wl = small_workload(n, T=T, H=H, topk=512, seed=41)
    L = synth.layer_inputs("reuse", wl.B, T, 0, H, 42, q_std=1.0)
    q = oracle.bf16_to_f64(L.q).reshape(wl.B, T, H, 512)
    e = np.linspace(-24, 24, H).round()
    q = q * (2.0 ** e)[None, None, :, None]
    L.q = np.asarray(torch.from_numpy(q.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()).view(np.uint16)
    wl.sm_scale = 2.0 ** -26
    idx = synth.random_topk(wl.B, T, 512, wl.n_entries, seed=43)
    out, _ = gpu_attention(wl, L, idx)
    assert np.isfinite(out).all()
    check_attention(oracle, wl, L, idx, out)


@pytest.mark.parametrize("T", [1, 8])
def test_attention_outlier_heavy(oracle, T):
    say(f"attention with 5% +-8 outliers and sharp logits, T={T}")
    n = [4096]
    wl = small_workload(n, T=T, H=64, topk=2048, seed=31)
    wl.kv_source = synth.kv_rows(4096, 32, outlier_frac=0.05)
    wl.sm_scale = 1.0 / 8.0
    L = synth.layer_inputs("reuse", 1, T, 0, 64, 33, q_std=1.0)
    idx = synth.random_topk(1, T, 2048, wl.n_entries, seed=34)
    out, _ = gpu_attention(wl, L, idx)
    check_attention(oracle, wl, L, idx, out)


def test_full_1m_b4_attention(oracle):
    say("attention 1M ctx B=4 H=64 k=2048 (Full-layer indices, 1% outliers)")
    wl = synth.workload("full_1m_b4")
    L = wl.layers[0]
    ref_tk, _, _ = oracle_index_full(oracle, wl, L)
    out, lse = gpu_attention(wl, L, ref_tk, with_lse=True)
    check_attention(oracle, wl, L, ref_tk, out, lse=lse)


def test_layer_step_graph_replays_match_eager(oracle):
    """A captured layer step (cache write, Full indexer, attention) replayed
    several times, with eager work and synchronizations between replays,
    gives the eager results on every replay; the eager result itself is
    checked against the oracle."""
    say("HIP graph of a layer step: 3 replays vs eager, n = [20000, 3001]")
    n = [20000, 3001]
    wl = small_workload(n, T=2, HI=16, H=16, topk=256, seed=21)
    L = wl.layers[0]
    B, T, H = wl.B, wl.T, wl.H
    kidx = dev(wl.kidx_pool)
    pt, ne = dev(wl.paging.page_table), dev(wl.n_entries)
    q_idx, w = dev(L.q_idx), dev(L.w)
    q = dev(L.q.view(np.int16), torch.bfloat16)
    swa = dev(L.swa)
    slots = wl.paging.all_slots()
    kv_pool = torch.zeros((wl.paging.n_pages, csa2.PAGE_BYTES), dtype=torch.uint8, device="cuda")
    csa2.quantize_kv(dev(wl.kv_source.view(np.int16), torch.bfloat16), dev(slots), kv_pool)
    last = np.cumsum(wl.n_entries) - 1
    rows = dev(wl.kv_source[last].view(np.int16), torch.bfloat16)
    rslots = dev(slots[last])
    out_topk = torch.empty((B, T, wl.topk), dtype=torch.int32, device="cuda")
    out_pool = torch.empty((B, T, wl.pool_blocks), dtype=torch.int32, device="cuda")
    out_pool_n = torch.empty((B, T), dtype=torch.int32, device="cuda")
    out = torch.empty((B, T, H, 512), dtype=torch.float32, device="cuda")
    ws_i, ws_a = csa2.Workspace(), csa2.Workspace()

    def step(strm):
        csa2.quantize_kv(rows, rslots, kv_pool, stream=strm)
        csa2.index_full(q_idx, w, kidx, pt, ne, wl.max_n, wl.topk, wl.pool_blocks, out_topk=out_topk,
                        out_pool=out_pool, out_pool_n=out_pool_n, ws=ws_i, stream=strm)
        csa2.sparse_attn(q, wl.sm_scale, kv_pool, pt, ne, out_topk, swa, out=out, ws=ws_a, stream=strm)

    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [host(x).copy() for x in (out_topk, out_pool, out_pool_n, out)]
    r_tk, r_pool, r_pn = oracle_index_full(oracle, wl, L)
    assert np.array_equal(ref[0], r_tk) and np.array_equal(ref[1], r_pool) and np.array_equal(ref[2], r_pn)

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step(torch.cuda.current_stream())
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        # eager work in between: scribble over the outputs, then replay
        out_topk.fill_(-7)
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [host(x) for x in (out_topk, out_pool, out_pool_n, out)]
        for a, b in zip(got, ref):
            assert np.array_equal(a, b), f"replay {rep} differs from the eager step"
