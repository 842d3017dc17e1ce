#!/usr/bin/env python3
"""CSA2 decode benchmark on one MI355X: layer-steps/s at 1M context.

One step is one decode layer of the CSA2 hot path over the whole batch, all
steps of it in the HIP library: the FP4 cache write of the step's new KV rows,
the Full-mode indexer (exact score scan over every visible entry, block-max
pool, top-k) and the sparse attention over the selected FP4 entries merged
with the 128-row FP8 window.  Inputs are seeded synthetic data of the 1M-token
workload (batch 4, 262,144 compressed entries per sequence, 64 indexer heads,
top-k 2,048, 64 query heads); caches are resident in HBM before timing, and
several copies are rotated so that the 256 MB Infinity Cache cannot serve a
step from the previous one.

Prints one JSON line: throughput, the dominant kernel's roofline (algorithmic
bytes / its average launch time, timed with HIP events on its launch stream),
and the CPU oracle timed on this host's cores on the same workload.

Other workloads (--workload), each printing its own JSON line:
  group_128k_b8     Full, Reindex and Reuse layer steps at 128K context, batch 8
  schedule_20l_b32  the 20-layer decoder schedule (Full at 20, Reindex at 24, 28,
                    32, 36, Reuse elsewhere), batch 32, 2 query tokens, ragged
                    32K..1M contexts, captured as one 20-layer step
  cache_write_1m    the FP4 cache write of 1,048,576 rows into permuted pages
  prefill_256t_1m   a 256-token prefill chunk (causal Full + Reindex + attention)
                    at the end of a 1M-token sequence
  full_8k_b1        the small Full layer (8K context, batch 1)
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "score_full_1m_b4_hbm_traffic.md")
SCAN_SRC = os.path.join(ROOT, "compressed_sparse_attention_mxfp4_amd", "csrc", "score.hip")
METRIC = "CSA2 decode layer-steps/s at 1M ctx; achieved HBM TB/s and % of peak"
DTYPE = "fp8/fp4 storage; f16-MFMA exact scores (int8-MFMA general path); f16-MFMA attention; fp32 softmax"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class HipEvents:
    """hipEvent_t pairs from the HIP runtime torch already loaded."""

    def __init__(self):
        self.rt = ctypes.CDLL("libamdhip64.so.7")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.rt.hipEventCreate(ctypes.byref(e)) == 0
            evs.append(e)
        return evs

    def elapsed_ms(self, a, b):
        """ms between two recorded events, or None (then the error is cleared, so that the
        next runtime call does not report it): e.g. a kernel the call did not launch."""
        f = ctypes.c_float()
        st = self.rt.hipEventElapsedTime(ctypes.byref(f), a, b)
        if st != 0:
            self.rt.hipGetLastError()
            return None
        return float(f.value)

    def destroy(self, evs):
        for e in evs:
            self.rt.hipEventDestroy(e)


class KernelTimer:
    """Per-launch durations of the library's kernels: around each library call,
    csa2_time_kernel registers a fresh event pair for every kernel that call
    launches, so each launch is bracketed on its own launch stream."""

    def __init__(self, csa2, ev):
        self.csa2, self.ev = csa2, ev
        self.spans = []          # (label, kernel name, start, stop)

    def call(self, label, kernels, fn):
        regs = []
        for name, kid in kernels.items():
            s, e = self.ev.create(2)
            self.csa2.lib().csa2_time_kernel(kid, s, e)
            regs.append((name, kid, s, e))
        fn()
        for name, kid, s, e in regs:
            self.csa2.lib().csa2_time_kernel(kid, None, None)
            self.spans.append((label, name, s, e))

    def collect(self, steps):
        """{label: {kernel: average us per step}} after the stream has drained."""
        out = {}
        for label, name, s, e in self.spans:
            d = out.setdefault(label, {})
            ms = self.ev.elapsed_ms(s, e)
            if ms is not None:       # None: the call did not launch this kernel
                d[name] = d.get(name, 0.0) + 1000.0 * ms / steps
            self.ev.destroy([s, e])
        self.spans = []
        return out


def kernel_ids(csa2):
    return {"full": {"score_full": csa2.K_SCORE_FULL, "select_full": csa2.K_SELECT_FULL},
            "reindex": {"score_reindex": csa2.K_SCORE_REINDEX, "select_reindex": csa2.K_SELECT_REINDEX},
            "attn": {"attn_split": csa2.K_ATTN_SPLIT, "attn_combine": csa2.K_ATTN_COMBINE}}


def algorithmic_bytes(wl, key_bytes=128):
    """Bytes the method must move per layer step (inputs read + outputs written);
    key_bytes: bytes per indexer key (128 E4M3, 68 MXFP4)."""
    n = int(np.sum(wl.n_entries))
    B, T, H, HI, k = wl.B, wl.T, wl.H, wl.HI, wl.topk
    scan = n * key_bytes + B * T * HI * (128 + 4)           # indexer keys + queries + weights
    idx_out = B * T * (k + wl.pool_blocks + 1) * 4           # top-k, pool, count
    attn = attention_bytes(wl)
    write = B * T * (1024 + 8 + 288)                         # new rows: bf16 in, slot, FP4 out
    return {"scan": scan, "step": scan + idx_out + attn + write}


def attention_bytes(wl, n_vis=None):
    """Selected FP4 entries + window rows + q in + out: one attention call."""
    B, T, H, k = wl.B, wl.T, wl.H, wl.topk
    if n_vis is None:
        sel = sum(min(k, int(n)) for n in wl.n_entries) * T
    else:
        sel = int(np.minimum(n_vis, k).sum())
    return sel * 288 + B * (127 + T) * 512 + B * T * H * 512 * (2 + 4)


def reindex_bytes(wl, pool_n, n_vis=None):
    """The Reindex scan's gathered pool keys (8 entries x 128 B per block) + queries + outputs."""
    B, T, HI, k = wl.B, wl.T, wl.HI, wl.topk
    pos = 0
    for b in range(B):
        for t in range(T):
            n = int(wl.n_entries[b]) if n_vis is None else min(int(wl.n_entries[b]), int(n_vis[b, t]))
            pn = int(pool_n[b, t])
            pos += min(pn * 8, n)
    return pos * 128 + B * T * HI * (128 + 4) + B * T * (wl.pool_blocks + 1 + k) * 4


def measured_traffic():
    """HBM bytes per score-scan launch from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE scaled by a plain copy's readings), or None
    when the scan kernel's source has changed since the counters were taken."""
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines()
                  if line.startswith(("traffic_bytes", "score_hip")))
    try:
        digest = hashlib.sha256(open(SCAN_SRC, "rb").read()).hexdigest()
    except OSError:
        return None
    if fields.get("score_hip_sha256", "").strip() != digest or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


def capture(torch, copies, step):
    """One captured HIP graph of `step(c, stream)` per cache copy c (on a side stream)."""
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                step(c, torch.cuda.current_stream())
            graphs.append(g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    return graphs


def time_steps(torch, ev, K, run_step):
    """Average ms per step over K steps, one event pair around all of them, and
    the host wall time per step."""
    whole = ev.create(2)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev.rt.hipEventRecord(whole[0], ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    for i in range(K):
        run_step(i)
    ev.rt.hipEventRecord(whole[1], ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = ev.elapsed_ms(whole[0], whole[1]) / K
    ev.destroy(whole)
    return ms, wall / K


def time_chained(torch, ev, K, chain, per, single):
    """Average ms per step over K steps replayed as graphs of `per` consecutive steps
    (chain()), the remainder as single-step graphs (single(i)); one event pair around all."""
    whole = ev.create(2)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev.rt.hipEventRecord(whole[0], ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    for _ in range(K // per):
        chain()
    for i in range(K % per):
        single(i)
    ev.rt.hipEventRecord(whole[1], ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = ev.elapsed_ms(whole[0], whole[1]) / K
    ev.destroy(whole)
    return ms, wall / K


def counters_driver(args):
    """Launch sequence for rocprofv3 counter runs: a plain 256 MiB device copy
    (calibrates FETCH_SIZE / WRITE_SIZE), then 3 times each: the Full indexer
    of the workload, the same over MXFP4 indexer keys, the cache write of all
    of the workload's rows (1,048,576 at 1M context), the fused RoPE + cache
    writes of those rows, the compressor forming that many entries at 4:1,
    the sparse attention over the indexer's top-k and the Reindex indexer over
    the Full indexer's pool."""
    import torch
    import compressed_sparse_attention_mxfp4_amd as csa2
    from compressed_sparse_attention_mxfp4_amd import synth
    csa2.load()
    n = 256 << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    wl = synth.workload(args.workload)
    L = wl.layers[0]
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, w, kidx, pt, ne = d(L.q_idx), d(L.w), d(wl.kidx_pool), d(wl.paging.page_table), d(wl.n_entries)
    ws = csa2.Workspace()
    for _ in range(3):
        topk, pool_, pool_n = csa2.index_full(q, w, kidx, pt, ne, wl.max_n, wl.topk, wl.pool_blocks, ws=ws)
    torch.cuda.synchronize()
    for _ in range(3):
        csa2.index_reindex(q, w, kidx, pt, ne, pool_, pool_n, wl.topk, ws=ws)
    torch.cuda.synchronize()
    # the same Full call over MXFP4 indexer keys (68 B per entry)
    kmx = d(synth.mxfp4_key_pool(wl.paging.n_pages, 45))
    for _ in range(3):
        csa2.index_full(q, w, kmx, pt, ne, wl.max_n, wl.topk, wl.pool_blocks, ws=ws, mxfp4=True)
    torch.cuda.synchronize()
    del kmx
    kv_src = d(wl.kv_source.view(np.int16)).view(torch.bfloat16)
    slots = d(wl.paging.all_slots())
    kv = torch.zeros((wl.paging.n_pages, csa2.PAGE_BYTES), dtype=torch.uint8, device="cuda")
    qa, swa = d(L.q.view(np.int16)).view(torch.bfloat16), d(L.swa)
    ws_a = csa2.Workspace()
    for _ in range(3):
        csa2.quantize_kv(kv_src, slots, kv)
    torch.cuda.synchronize()
    # fused RoPE + cache writes of the same rows, indexer keys too, row j at position j
    R = kv_src.shape[0]
    ki_src = d(synth.kidx_rows(R, 46).view(np.int16)).view(torch.bfloat16)
    pos, table = d(np.arange(R, dtype=np.int64)), d(synth.rope_table(R))
    kip = torch.zeros((wl.paging.n_pages, csa2.PAGE, csa2.DI), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        csa2.rope_write_caches(kv_src, ki_src, pos, table, slots, kv, kip)
    torch.cuda.synchronize()
    del ki_src, pos, table, kip
    # the compressor at 4:1 over the source positions of the same entries (4 x the rows)
    gen = torch.Generator(device="cuda").manual_seed(47)
    csrc = torch.randn((4 * R, csa2.D), generator=gen, device="cuda").to(torch.bfloat16)
    zsrc = torch.randn((4 * R, csa2.D), generator=gen, device="cuda").to(torch.bfloat16)
    ent = torch.empty((R, csa2.D), dtype=torch.bfloat16, device="cuda")
    for _ in range(3):
        csa2.compress(csrc, zsrc, 4, out=ent)
    torch.cuda.synchronize()
    del csrc, zsrc, ent
    for _ in range(3):
        csa2.sparse_attn(qa, wl.sm_scale, kv, pt, ne, topk, swa, ws=ws_a)
    torch.cuda.synchronize()
    log("counters driver done")
    return 0


def cpu_baseline(wl, min_seconds=12.0, max_reps=40, kidx_mx=None):
    """The oracle, as it stands, on the same layer step; all host cores it uses."""
    import oracle
    oracle.build(force=False)
    L = wl.layers[0]
    offs = np.concatenate([[0], np.cumsum(wl.n_entries)[:-1]])
    reps, t0 = 0, time.perf_counter()
    while True:
        if kidx_mx is not None:
            tk, _, _ = oracle.index_full_mxfp4(L.q_idx, L.w, kidx_mx, wl.paging.page_table, wl.n_entries,
                                               wl.topk, wl.pool_blocks)
        else:
            tk, _, _ = oracle.index_full(L.q_idx, L.w, wl.kidx_pool, wl.paging.page_table, wl.n_entries,
                                         wl.topk, wl.pool_blocks)
        for b in range(wl.B):
            for t in range(wl.T):
                sel = tk[b, t][tk[b, t] >= 0].astype(np.int64)
                oracle.sparse_attn_from_rows(L.q[b, t], wl.sm_scale, wl.kv_source[offs[b] + sel],
                                             L.swa[b, t:t + 128])
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= max_reps:
            break
    return {"value": reps / el, "unit": "layer-steps/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"whole layer step of the same workload (index over {int(np.sum(wl.n_entries))} "
                      f"entries x {wl.T} token(s), top-k, pool, attention for {wl.B * wl.T} queries), "
                      f"{reps} repetitions in {el:.1f} s"}


def cpu_baseline_schedule(wl, sample_layers=(20, 21, 24)):
    """The oracle on a bounded sample of the 20-layer step: the Full layer (index + attention),
    one Reuse attention and one Reindex layer over the whole batch, scaled to the 20-layer step
    by the per-mode counts (1 Full, 4 Reindex, 15 Reuse)."""
    import oracle
    oracle.build(force=False)
    offs = np.concatenate([[0], np.cumsum(wl.n_entries)[:-1]])
    by = {20 + i: L for i, L in enumerate(wl.layers)}

    def attend(L, tk):
        for b in range(wl.B):
            for t in range(wl.T):
                sel = tk[b, t][tk[b, t] >= 0].astype(np.int64)
                oracle.sparse_attn_from_rows(L.q[b, t], wl.sm_scale, wl.kv_source[offs[b] + sel],
                                             L.swa[b, t:t + 128])

    t0 = time.perf_counter()
    L = by[20]
    tk, pool_, pool_n = oracle.index_full(L.q_idx, L.w, wl.kidx_pool, wl.paging.page_table, wl.n_entries,
                                          wl.topk, wl.pool_blocks)
    t_full_idx = time.perf_counter() - t0
    attend(L, tk)
    t1 = time.perf_counter()
    t_attn = t1 - t0 - t_full_idx
    R = by[24]
    rtk = oracle.index_reindex(R.q_idx, R.w, wl.kidx_pool, wl.paging.page_table, wl.n_entries, pool_, pool_n,
                               wl.topk)
    t_re_idx = time.perf_counter() - t1
    step = t_full_idx + 4 * t_re_idx + 20 * t_attn
    el = time.perf_counter() - t0
    return {"value": 1.0 / step, "unit": "20-layer steps/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": f"the Full layer (index over {int(np.sum(wl.n_entries))} entries x {wl.T} tokens + "
                      f"attention for {wl.B * wl.T} queries) and one Reindex index, timed once ({el:.1f} s) and "
                      f"scaled to 1 Full index + 4 Reindex indexes + 20 attentions"}


def _setup(args):
    import torch
    import compressed_sparse_attention_mxfp4_amd as csa2
    if not os.path.exists(csa2.LIB_PATH):
        from compressed_sparse_attention_mxfp4_amd import build
        build.build()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    csa2.load()
    return torch, csa2, torch.device("cuda:0")


def _uploader(torch, dev):
    def up(a, dtype=None):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(dtype) if dtype is not None else t).to(dev)
    return up


def new_rows_for_step(wl, up, torch, slots_all):
    """The step's cache write: one fresh bf16 row per sequence (seeded, not the row the cache was
    built from) into the slot of that sequence's newest entry."""
    from compressed_sparse_attention_mxfp4_amd import synth
    last = np.cumsum(wl.n_entries) - 1
    rows = up(synth.kv_rows(wl.B, 99, outlier_frac=0.01).view(np.int16), torch.bfloat16)
    return rows, slots_all[torch.from_numpy(last).to(rows.device)].contiguous()


def check_fused_write(torch, csa2, kv_pool, rows, slots, n_pages):
    """The fused cache write landed: the pool bytes (codes and scales) at the new slots equal a
    separate csa2_quantize_kv of the same rows."""
    ref = torch.zeros((n_pages, csa2.PAGE_BYTES), dtype=torch.uint8, device=kv_pool.device)
    csa2.quantize_kv(rows, slots, ref)
    for s in slots.cpu().numpy().tolist():
        p, o = s // 64, s % 64
        for lo, hi in ((o * 256, (o + 1) * 256), (16384 + o * 32, 16384 + (o + 1) * 32)):
            assert torch.equal(kv_pool[p, lo:hi], ref[p, lo:hi]), f"fused cache write missing at slot {s}"


# ---------------------------------------------------------------- the 1M-context layer step (headline)
def bench_layer(args):
    torch, csa2, dev = _setup(args)
    from compressed_sparse_attention_mxfp4_amd import synth
    t0 = time.perf_counter()
    wl = synth.workload(args.workload)
    L = wl.layers[0]
    if args.score_path == "general-q":
        # indexer queries N(0, 64^2): every row has some |q| >= 32, so the scan scores it on the
        # int8 three-limb path
        L.q_idx = synth.fp8_normal(L.q_idx.shape, 901, std=64.0)
    elif args.score_path == "general-k":
        # indexer keys N(0, 4^2): every entry has sum k^2 > 500, so every chunk takes the int8 path
        wl.kidx_pool = synth.fp8_normal(wl.kidx_pool.shape, 902, std=4.0)
    log(f"workload {args.workload} generated in {time.perf_counter() - t0:.1f} s")
    up = _uploader(torch, dev)
    pt, ne = up(wl.paging.page_table), up(wl.n_entries)
    q_idx, w = up(L.q_idx), up(L.w)
    q, swa = up(L.q.view(np.int16), torch.bfloat16), up(L.swa)
    kv_src = up(wl.kv_source.view(np.int16), torch.bfloat16)
    slots = up(wl.paging.all_slots())
    mx = args.kidx_format == "mxfp4"
    kidx_mx = synth.mxfp4_key_pool(wl.paging.n_pages, 45) if mx else None
    kidx0 = up(kidx_mx if mx else wl.kidx_pool)
    kv0 = torch.zeros((wl.paging.n_pages, csa2.PAGE_BYTES), dtype=torch.uint8, device=dev)
    csa2.quantize_kv(kv_src, slots, kv0)
    kidx = [kidx0] + [kidx0.clone() for _ in range(args.copies - 1)]
    kvp = [kv0] + [kv0.clone() for _ in range(args.copies - 1)]
    new_rows, new_slots = new_rows_for_step(wl, up, torch, slots)
    del kv_src
    B, T, H = wl.B, wl.T, wl.H
    out_topk = torch.empty((B, T, wl.topk), dtype=torch.int32, device=dev)
    out_pool = torch.empty((B, T, wl.pool_blocks), dtype=torch.int32, device=dev)
    out_pool_n = torch.empty((B, T), dtype=torch.int32, device=dev)
    out = torch.empty((B, T, H, 512), dtype=torch.float32, device=dev)
    ws_i, ws_a = csa2.Workspace(), csa2.Workspace()
    stream = torch.cuda.current_stream()
    ids = kernel_ids(csa2)

    def step(i, strm, timer=None):
        c = i % args.copies
        # the cache write rides in the indexer's launches (csa2_index_full[_mxfp4]_write); it
        # lands before the attention, which reads the new entries
        f = lambda: csa2.index_full(q_idx, w, kidx[c], pt, ne, wl.max_n, wl.topk, wl.pool_blocks,
                                    out_topk=out_topk, out_pool=out_pool, out_pool_n=out_pool_n, ws=ws_i,
                                    stream=strm, mxfp4=mx, write=(new_rows, new_slots, kvp[c]))
        a = lambda: csa2.sparse_attn(q, wl.sm_scale, kvp[c], pt, ne, out_topk, swa, out=out, ws=ws_a, stream=strm)
        if timer is None:
            f()
            a()
        else:
            timer.call("index", ids["full"], f)
            timer.call("attn", ids["attn"], a)

    for i in range(args.warmup):
        step(i, stream)
    torch.cuda.synchronize()
    for c in range(min(args.copies, args.warmup)):
        check_fused_write(torch, csa2, kvp[c], new_rows, new_slots, wl.paging.n_pages)
    ev = HipEvents()
    K = args.steps

    # ---- pass 1: per-kernel durations (eager launches, an event pair around each launch)
    timer = KernelTimer(csa2, ev)
    torch.cuda.synchronize()
    for i in range(K):
        step(args.warmup + i, stream, timer)
    torch.cuda.synchronize()
    per = timer.collect(K)
    kern_us = {**per["index"], **per["attn"]}
    kern_us.setdefault("attn_combine", 0.0)
    eager_ref = out_topk.clone(), out.clone()

    # ---- pass 2: whole steps, timed with one event pair around K steps
    graphs = None
    if not args.eager:
        # one captured step per cache copy; the library makes no allocation or memset
        graphs = capture(torch, args.copies, lambda c, s: step(c, s))
        # a replay reproduces the eager step (same copy as the last eager step)
        last = (args.warmup + K - 1) % args.copies
        graphs[last].replay()
        torch.cuda.synchronize()
        assert torch.equal(out_topk, eager_ref[0]) and torch.equal(out, eager_ref[1]), \
            "graph replay differs from the eager step"
        for i in range(args.warmup):
            graphs[i % args.copies].replay()
        torch.cuda.synchronize()
        # the same steps captured `steps_per_graph` at a time (step j on cache copy j mod copies),
        # as a decode forward captures its consecutive layers in one graph: the gap the GPU leaves
        # between two graph launches is paid once per graph
        spg = args.steps_per_graph
        chain = capture(torch, 1, lambda _c, s: [step(c, s) for c in range(spg)])[0]
        step(spg - 1, stream)
        torch.cuda.synchronize()
        ref_last = out_topk.clone(), out.clone()
        chain.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_topk, ref_last[0]) and torch.equal(out, ref_last[1]), \
            "chained graph replay differs from the eager step"
        for _ in range(max(1, args.warmup // spg)):
            chain.replay()
        torch.cuda.synchronize()

    def run_step(i):
        if graphs is not None:
            graphs[i % args.copies].replay()
        else:
            step(i, stream)

    ms_single, wall_single = time_steps(torch, ev, K, run_step)
    if graphs is not None:
        ms_per_step, wall = time_chained(torch, ev, K, chain.replay, spg,
                                         lambda i: graphs[i % args.copies].replay())
    else:
        ms_per_step, wall = ms_single, wall_single
    value = 1000.0 / ms_per_step
    nbytes = algorithmic_bytes(wl, 68 if mx else 128)
    scan_gbs = nbytes["scan"] / (kern_us["score_full"] * 1e-6) / 1e9
    step_gbs = nbytes["step"] / (ms_per_step * 1e-3) / 1e9
    log(f"{K} steps ({'eager' if graphs is None else f'graph replay, {args.steps_per_graph} steps per graph'}): "
        f"{ms_per_step * 1000:.1f} us/step (wall {wall * 1e6:.1f} us/step); "
        + ("" if graphs is None else f"one step per graph {ms_single * 1000:.1f} us/step; ")
        + "kernels us: " + ", ".join(f"{k}={v:.1f}" for k, v in kern_us.items()))

    result = {
        "metric": METRIC, "value": round(value, 2), "unit": "layer-steps/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": DTYPE, "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "query_tokens": T,
                   "context_tokens": int(wl.max_n) * 4, "entries_per_seq": int(wl.max_n),
                   "indexer_heads": wl.HI, "heads": H, "topk": wl.topk, "pool_blocks": wl.pool_blocks,
                   "indexer_key_format": args.kidx_format, "cache_copies_rotated": args.copies,
                   "score_path": args.score_path,
                   "launch": "eager" if graphs is None else "hip_graph_replay",
                   "steps_per_graph": None if graphs is None else args.steps_per_graph},
        "ms_per_step_one_step_per_graph": None if graphs is None else round(ms_single, 5),
        "hbm_tb_s": round(step_gbs / 1000.0, 3),
        "hbm_frac_of_peak": round(step_gbs / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": nbytes["step"],
        "kernel_avg_us": {k: round(v, 2) for k, v in kern_us.items()},
        "roofline": {"kernel": "score_kernel (Full-mode exact score scan)", "bound": "hbm",
                     "achieved": round(scan_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(scan_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None if (mx or args.workload != "full_1m_b4" or args.score_path != "fast")
                     else measured_traffic(),
                     "algorithmic_bytes_per_launch": nbytes["scan"]},
    }
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        result["cpu_baseline"] = cpu_baseline(wl, kidx_mx=kidx_mx)
        log(f"cpu baseline in {time.perf_counter() - t0:.1f} s")
    print(json.dumps(result), flush=True)
    return 0


# ---------------------------------------------------------------- multi-layer workloads
def _mode_result(args, metric, value, unit, ms, K, config, extra):
    r = {"metric": metric, "value": round(value, 3), "unit": unit, "n_gpus": 1, "steps": K,
         "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
         "vs_baseline": None, "dtype": DTYPE, "data": "synthetic", "config": config}
    r.update(extra)
    return r


def _roof(kernel, nbytes, us):
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None, "algorithmic_bytes_per_launch": int(nbytes)}


def bench_schedule(args):
    """The 20-layer decoder schedule as one captured step: layer 20 Full (with the step's cache
    write), layers 24/28/32/36 Reindex over layer 20's pool, every layer its own attention (Reuse
    layers with the latest Full/Reindex indices)."""
    torch, csa2, dev = _setup(args)
    from compressed_sparse_attention_mxfp4_amd import synth
    t0 = time.perf_counter()
    wl = synth.workload("schedule_20l_b32")
    log(f"workload schedule_20l_b32 generated in {time.perf_counter() - t0:.1f} s "
        f"(sum n = {int(wl.n_entries.sum())}, max n = {wl.max_n})")
    up = _uploader(torch, dev)
    B, T, H, k = wl.B, wl.T, wl.H, wl.topk
    pt, ne = up(wl.paging.page_table), up(wl.n_entries)
    slots = up(wl.paging.all_slots())
    kv_src = up(wl.kv_source.view(np.int16), torch.bfloat16)
    kv0 = torch.zeros((wl.paging.n_pages, csa2.PAGE_BYTES), dtype=torch.uint8, device=dev)
    csa2.quantize_kv(kv_src, slots, kv0)
    del kv_src
    copies = max(1, min(args.copies, 2))      # each copy is ~1 GB: 2 copies exceed the 256 MB MALL
    kidx = [up(wl.kidx_pool)] + [up(wl.kidx_pool) for _ in range(copies - 1)]
    kvp = [kv0] + [kv0.clone() for _ in range(copies - 1)]
    new_rows, new_slots = new_rows_for_step(wl, up, torch, slots)
    layers = []
    for i, L in enumerate(wl.layers):
        layers.append({"li": 20 + i, "mode": L.mode,
                       "q_idx": up(L.q_idx) if L.q_idx is not None else None,
                       "w": up(L.w) if L.w is not None else None,
                       "q": up(L.q.view(np.int16), torch.bfloat16), "swa": up(L.swa),
                       "out": torch.empty((B, T, H, 512), dtype=torch.float32, device=dev)})
    tk_full = torch.empty((B, T, k), dtype=torch.int32, device=dev)
    pool_ = torch.empty((B, T, wl.pool_blocks), dtype=torch.int32, device=dev)
    pool_n = torch.empty((B, T), dtype=torch.int32, device=dev)
    tk_re = [torch.empty((B, T, k), dtype=torch.int32, device=dev) for _ in range(4)]
    ws_i, ws_a = csa2.Workspace(), csa2.Workspace()
    ids = kernel_ids(csa2)
    stream = torch.cuda.current_stream()

    def step(i, strm, timer=None):
        c = i % copies
        cur = None
        r = 0
        for Ld in layers:
            if Ld["mode"] == "full":
                fn = lambda: csa2.index_full(Ld["q_idx"], Ld["w"], kidx[c], pt, ne, wl.max_n, k, wl.pool_blocks,
                                             out_topk=tk_full, out_pool=pool_, out_pool_n=pool_n, ws=ws_i,
                                             stream=strm, write=(new_rows, new_slots, kvp[c]))
                timer.call("full_index", ids["full"], fn) if timer else fn()
                cur = tk_full
            elif Ld["mode"] == "reindex":
                dst = tk_re[r]
                fn = lambda: csa2.index_reindex(Ld["q_idx"], Ld["w"], kidx[c], pt, ne, pool_, pool_n, k,
                                                out_topk=dst, ws=ws_i, stream=strm)
                timer.call("reindex_index", ids["reindex"], fn) if timer else fn()
                cur = dst
                r += 1
            fa = lambda: csa2.sparse_attn(Ld["q"], wl.sm_scale, kvp[c], pt, ne, cur, Ld["swa"], out=Ld["out"],
                                          ws=ws_a, stream=strm)
            label = {"full": "full_attn", "reindex": "reindex_attn", "reuse": "reuse_attn"}[Ld["mode"]]
            timer.call(label, ids["attn"], fa) if timer else fa()

    for i in range(args.warmup):
        step(i, stream)
    torch.cuda.synchronize()
    for c in range(min(copies, args.warmup)):
        check_fused_write(torch, csa2, kvp[c], new_rows, new_slots, wl.paging.n_pages)
    ev = HipEvents()
    K = args.steps
    timer = KernelTimer(csa2, ev)
    for i in range(K):
        step(args.warmup + i, stream, timer)
    torch.cuda.synchronize()
    per = timer.collect(K)
    ref = [Ld["out"].clone() for Ld in layers], [t.clone() for t in tk_re], tk_full.clone()
    graphs = capture(torch, copies, lambda c, s: step(c, s))
    last = (args.warmup + K - 1) % copies
    graphs[last].replay()
    torch.cuda.synchronize()
    assert torch.equal(tk_full, ref[2]) and all(torch.equal(a, b) for a, b in zip(tk_re, ref[1])) and \
        all(torch.equal(Ld["out"], o) for Ld, o in zip(layers, ref[0])), "graph replay differs from the eager step"
    for i in range(args.warmup):
        graphs[i % copies].replay()
    ms, wall = time_steps(torch, ev, K, lambda i: graphs[i % copies].replay())
    pn = pool_n.cpu().numpy()
    mode_us = {
        "full_index": sum(per["full_index"].values()),
        "reindex_index_each": sum(per["reindex_index"].values()) / 4,
        "attention_each": (sum(per["full_attn"].values()) + sum(per["reindex_attn"].values())
                           + sum(per["reuse_attn"].values())) / 20,
    }
    mode_us["full_layer"] = mode_us["full_index"] + sum(per["full_attn"].values())
    mode_us["reindex_layer"] = mode_us["reindex_index_each"] + sum(per["reindex_attn"].values()) / 4
    mode_us["reuse_layer"] = sum(per["reuse_attn"].values()) / 15
    kern = {}
    for label, d in per.items():
        for name, v in d.items():
            kern[f"{label}.{name}"] = round(v, 2)
    scan_bytes = int(wl.n_entries.sum()) * 128 + B * T * wl.HI * 132
    re_bytes = reindex_bytes(wl, pn)
    at_bytes = attention_bytes(wl)
    step_bytes = scan_bytes + 4 * re_bytes + 20 * at_bytes + B * (1024 + 8 + 288)
    log(f"20-layer step: {ms * 1000:.1f} us (wall {wall * 1e6:.1f} us); per mode us: "
        + ", ".join(f"{a}={b:.1f}" for a, b in mode_us.items()))
    result = _mode_result(
        args, "CSA2 20-layer decoder steps/s (Full 20, Reindex 24/28/32/36, Reuse elsewhere)", 1000.0 / ms,
        "20-layer steps/s", ms, K,
        {"workload": "schedule_20l_b32", "batch": B, "query_tokens": T, "entries_per_seq_min": int(wl.n_entries.min()),
         "entries_per_seq_max": int(wl.max_n), "entries_total": int(wl.n_entries.sum()), "indexer_heads": wl.HI,
         "heads": H, "topk": k, "pool_blocks": wl.pool_blocks, "layers": 20, "cache_copies_rotated": copies,
         "launch": "hip_graph_replay"},
        {"mode_us": {a: round(b, 2) for a, b in mode_us.items()}, "kernel_avg_us_per_step": kern,
         "algorithmic_bytes_per_step": int(step_bytes),
         "hbm_tb_s": round(step_bytes / (ms * 1e-3) / 1e12, 3),
         "roofline": _roof("score_kernel (Full-mode exact score scan)", scan_bytes,
                           per["full_index"]["score_full"]),
         "roofline_reindex_scan": _roof("score_kernel (Reindex pool scan)", re_bytes,
                                        per["reindex_index"]["score_reindex"] / 4),
         "roofline_attention": _roof("attn_split + attn_combine", at_bytes, mode_us["attention_each"])})
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_schedule(wl)
    print(json.dumps(result), flush=True)
    return 0


def bench_group(args):
    """Full, Reindex and Reuse layer steps of the 128K-context batch-8 group, each its own
    captured step, timed separately."""
    torch, csa2, dev = _setup(args)
    from compressed_sparse_attention_mxfp4_amd import synth
    wl = synth.workload("group_128k_b8")
    up = _uploader(torch, dev)
    B, T, H, k = wl.B, wl.T, wl.H, wl.topk
    pt, ne = up(wl.paging.page_table), up(wl.n_entries)
    slots = up(wl.paging.all_slots())
    kv_src = up(wl.kv_source.view(np.int16), torch.bfloat16)
    kv0 = torch.zeros((wl.paging.n_pages, csa2.PAGE_BYTES), dtype=torch.uint8, device=dev)
    csa2.quantize_kv(kv_src, slots, kv0)
    del kv_src
    kidx = [up(wl.kidx_pool)] + [up(wl.kidx_pool) for _ in range(args.copies - 1)]
    kvp = [kv0] + [kv0.clone() for _ in range(args.copies - 1)]
    new_rows, new_slots = new_rows_for_step(wl, up, torch, slots)
    full, reidx, reuse = wl.layers
    F = {"q_idx": up(full.q_idx), "w": up(full.w), "q": up(full.q.view(np.int16), torch.bfloat16), "swa": up(full.swa)}
    R = {"q_idx": up(reidx.q_idx), "w": up(reidx.w), "q": up(reidx.q.view(np.int16), torch.bfloat16),
         "swa": up(reidx.swa)}
    U = {"q": up(reuse.q.view(np.int16), torch.bfloat16), "swa": up(reuse.swa)}
    tk = torch.empty((B, T, k), dtype=torch.int32, device=dev)
    pool_ = torch.empty((B, T, wl.pool_blocks), dtype=torch.int32, device=dev)
    pool_n = torch.empty((B, T), dtype=torch.int32, device=dev)
    rtk = torch.empty((B, T, k), dtype=torch.int32, device=dev)
    out = torch.empty((B, T, H, 512), dtype=torch.float32, device=dev)
    ws_i, ws_a = csa2.Workspace(), csa2.Workspace()
    ids = kernel_ids(csa2)

    def full_step(c, strm, timer=None):
        f = lambda: csa2.index_full(F["q_idx"], F["w"], kidx[c], pt, ne, wl.max_n, k, wl.pool_blocks, out_topk=tk,
                                    out_pool=pool_, out_pool_n=pool_n, ws=ws_i, stream=strm,
                                    write=(new_rows, new_slots, kvp[c]))
        a = lambda: csa2.sparse_attn(F["q"], wl.sm_scale, kvp[c], pt, ne, tk, F["swa"], out=out, ws=ws_a, stream=strm)
        timer.call("full_index", ids["full"], f) if timer else f()
        timer.call("full_attn", ids["attn"], a) if timer else a()

    def reindex_step(c, strm, timer=None):
        f = lambda: csa2.index_reindex(R["q_idx"], R["w"], kidx[c], pt, ne, pool_, pool_n, k, out_topk=rtk, ws=ws_i,
                                       stream=strm)
        a = lambda: csa2.sparse_attn(R["q"], wl.sm_scale, kvp[c], pt, ne, rtk, R["swa"], out=out, ws=ws_a,
                                     stream=strm)
        timer.call("reindex_index", ids["reindex"], f) if timer else f()
        timer.call("reindex_attn", ids["attn"], a) if timer else a()

    def reuse_step(c, strm, timer=None):
        a = lambda: csa2.sparse_attn(U["q"], wl.sm_scale, kvp[c], pt, ne, rtk, U["swa"], out=out, ws=ws_a,
                                     stream=strm)
        timer.call("reuse_attn", ids["attn"], a) if timer else a()

    stream = torch.cuda.current_stream()
    steps = {"full": full_step, "reindex": reindex_step, "reuse": reuse_step}
    for i in range(args.warmup):
        for fn in steps.values():
            fn(i % args.copies, stream)
    torch.cuda.synchronize()
    ev = HipEvents()
    K = args.steps
    timer = KernelTimer(csa2, ev)
    for i in range(K):
        for fn in steps.values():
            fn(i % args.copies, stream, timer)
    torch.cuda.synchronize()
    per = timer.collect(K)
    ms = {}
    for name, fn in steps.items():
        graphs = capture(torch, args.copies, lambda c, s, fn=fn: fn(c, s))
        for i in range(args.warmup):
            graphs[i % args.copies].replay()
        ms[name], _ = time_steps(torch, ev, K, lambda i, g=graphs: g[i % args.copies].replay())
    pn = pool_n.cpu().numpy()
    scan_bytes = int(wl.n_entries.sum()) * 128 + B * T * wl.HI * 132
    re_bytes = reindex_bytes(wl, pn)
    at_bytes = attention_bytes(wl)
    group_ms = ms["full"] + ms["reindex"] + ms["reuse"]
    kern = {f"{label}.{name}": round(v, 2) for label, d in per.items() for name, v in d.items()}
    log("group 128K B=8 layer steps us: " + ", ".join(f"{a}={b * 1000:.1f}" for a, b in ms.items()))
    result = _mode_result(
        args, "CSA2 Full+Reindex+Reuse group steps/s at 128K ctx, batch 8", 1000.0 / group_ms, "group steps/s",
        group_ms, K,
        {"workload": "group_128k_b8", "batch": B, "query_tokens": T, "entries_per_seq": int(wl.max_n),
         "indexer_heads": wl.HI, "heads": H, "topk": k, "pool_blocks": wl.pool_blocks,
         "cache_copies_rotated": args.copies, "launch": "hip_graph_replay"},
        {"layer_step_us": {a: round(b * 1000, 2) for a, b in ms.items()}, "kernel_avg_us": kern,
         "algorithmic_bytes": {"full_layer": scan_bytes + at_bytes, "reindex_layer": re_bytes + at_bytes,
                               "reuse_layer": at_bytes},
         "roofline": _roof("score_kernel (Reindex pool scan)", re_bytes, per["reindex_index"]["score_reindex"]),
         "roofline_full_scan": _roof("score_kernel (Full-mode exact score scan)", scan_bytes,
                                     per["full_index"]["score_full"]),
         "roofline_attention": _roof("attn_split + attn_combine", at_bytes,
                                     sum(per["reuse_attn"].values()))})
    print(json.dumps(result), flush=True)
    return 0


def bench_cache_write(args):
    """The FP4 cache write of 1,048,576 post-RoPE rows into permuted 64-entry pages."""
    torch, csa2, dev = _setup(args)
    from compressed_sparse_attention_mxfp4_amd import synth
    x, slots, n_pages = synth.cache_write_rows()
    up = _uploader(torch, dev)
    R = x.shape[0]
    copies = max(1, min(args.copies, 2))
    xs = [up(x.view(np.int16), torch.bfloat16) for _ in range(copies)]
    sl = up(slots)
    pools = [torch.zeros((n_pages, csa2.PAGE_BYTES), dtype=torch.uint8, device=dev) for _ in range(copies)]
    for i in range(args.warmup):
        csa2.quantize_kv(xs[i % copies], sl, pools[i % copies])
    torch.cuda.synchronize()
    ev = HipEvents()
    K = args.steps
    timer = KernelTimer(csa2, ev)
    for i in range(K):
        timer.call("write", {"quantize": csa2.K_QUANTIZE},
                   lambda: csa2.quantize_kv(xs[i % copies], sl, pools[i % copies]))
    torch.cuda.synchronize()
    us = timer.collect(K)["write"]["quantize"]
    ms, _ = time_steps(torch, ev, K, lambda i: csa2.quantize_kv(xs[i % copies], sl, pools[i % copies]))
    nbytes = R * (1024 + 8 + 288)
    log(f"cache write of {R} rows: {us:.1f} us per launch, {ms * 1000:.1f} us per call")
    result = _mode_result(args, "CSA2 FP4 cache-write rows/s (E2M1 + E4M3 per 16 ch, paged)", R / (ms * 1e-3),
                          "rows/s", ms, K,
                          {"workload": "cache_write_1m", "rows": R, "pages": n_pages, "page_order": "seeded permutation",
                           "buffers_rotated": copies},
                          {"kernel_avg_us": {"quantize": round(us, 2)}, "algorithmic_bytes_per_call": nbytes,
                           "roofline": _roof("quantize_kv_kernel", nbytes, us)})
    print(json.dumps(result), flush=True)
    return 0


def bench_prefill(args):
    """A 256-token prefill chunk at the end of a 1M-token sequence: the causal Full indexer,
    attention over its top-k, the causal Reindex indexer over its pool, attention again."""
    torch, csa2, dev = _setup(args)
    from compressed_sparse_attention_mxfp4_amd import synth
    wl = synth.workload("prefill_256t_1m")
    up = _uploader(torch, dev)
    B, T, H, k = wl.B, wl.T, wl.H, wl.topk
    n_vis = synth.prefill_counts(wl.n_entries, T)
    pt, ne, nv = up(wl.paging.page_table), up(wl.n_entries), up(n_vis)
    slots = up(wl.paging.all_slots())
    kv_src = up(wl.kv_source.view(np.int16), torch.bfloat16)
    kv = torch.zeros((wl.paging.n_pages, csa2.PAGE_BYTES), dtype=torch.uint8, device=dev)
    csa2.quantize_kv(kv_src, slots, kv)
    del kv_src
    kidx = up(wl.kidx_pool)
    full, reidx = wl.layers
    F = {"q_idx": up(full.q_idx), "w": up(full.w), "q": up(full.q.view(np.int16), torch.bfloat16), "swa": up(full.swa)}
    R = {"q_idx": up(reidx.q_idx), "w": up(reidx.w), "q": up(reidx.q.view(np.int16), torch.bfloat16),
         "swa": up(reidx.swa)}
    tk = torch.empty((B, T, k), dtype=torch.int32, device=dev)
    pool_ = torch.empty((B, T, wl.pool_blocks), dtype=torch.int32, device=dev)
    pool_n = torch.empty((B, T), dtype=torch.int32, device=dev)
    rtk = torch.empty((B, T, k), dtype=torch.int32, device=dev)
    out = torch.empty((B, T, H, 512), dtype=torch.float32, device=dev)
    ws_i, ws_a = csa2.Workspace(), csa2.Workspace()
    ids = kernel_ids(csa2)

    def step(strm, timer=None):
        calls = [("full_index", ids["full"], lambda: csa2.index_full(
                     F["q_idx"], F["w"], kidx, pt, ne, wl.max_n, k, wl.pool_blocks, out_topk=tk, out_pool=pool_,
                     out_pool_n=pool_n, ws=ws_i, stream=strm, n_visible=nv)),
                 ("full_attn", ids["attn"], lambda: csa2.sparse_attn(F["q"], wl.sm_scale, kv, pt, ne, tk, F["swa"],
                                                                     out=out, ws=ws_a, stream=strm)),
                 ("reindex_index", ids["reindex"], lambda: csa2.index_reindex(
                     R["q_idx"], R["w"], kidx, pt, ne, pool_, pool_n, k, out_topk=rtk, ws=ws_i, stream=strm,
                     n_visible=nv)),
                 ("reindex_attn", ids["attn"], lambda: csa2.sparse_attn(R["q"], wl.sm_scale, kv, pt, ne, rtk,
                                                                        R["swa"], out=out, ws=ws_a, stream=strm))]
        for label, kids, fn in calls:
            timer.call(label, kids, fn) if timer else fn()

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        step(stream)
    torch.cuda.synchronize()
    ev = HipEvents()
    K = args.steps
    timer = KernelTimer(csa2, ev)
    for _ in range(K):
        step(stream, timer)
    torch.cuda.synchronize()
    per = timer.collect(K)
    graphs = capture(torch, 1, lambda c, s: step(s))
    for _ in range(args.warmup):
        graphs[0].replay()
    ms, _ = time_steps(torch, ev, K, lambda i: graphs[0].replay())
    pn = pool_n.cpu().numpy()
    scan_bytes = int(wl.n_entries.sum()) * 128 + B * T * wl.HI * 132
    flops = 2.0 * 2 * wl.HI * 128 * float(np.minimum(n_vis, wl.n_entries[:, None]).sum())  # two f16 limbs
    us_scan = per["full_index"]["score_full"]
    tflops = flops / (us_scan * 1e-6) / 1e12
    kern = {f"{label}.{name}": round(v, 2) for label, d in per.items() for name, v in d.items()}
    log(f"prefill chunk T={T}: {ms * 1000:.1f} us per Full+Reindex pair; scan {us_scan:.1f} us = {tflops:.0f} TFLOP/s")
    result = _mode_result(
        args, "CSA2 prefill-chunk query tokens/s (causal Full + Reindex layers with attention)", T * B / (ms * 1e-3),
        "tokens/s", ms, K,
        {"workload": "prefill_256t_1m", "batch": B, "query_tokens": T, "entries_per_seq": int(wl.max_n),
         "indexer_heads": wl.HI, "heads": H, "topk": k, "pool_blocks": wl.pool_blocks, "launch": "hip_graph_replay"},
        {"kernel_avg_us": kern,
         "roofline": {"kernel": "score_kernel (Full-mode causal scan, 256 tokens)", "bound": "mfma",
                      "achieved": round(tflops, 1), "peak": 2500.0, "unit": "TFLOP/s",
                      "frac": round(tflops / 2500.0, 4), "traffic": None,
                      "note": "f16 MFMA flops of the two-limb exact products (2 x 2 x HI x 128 per visible "
                              "entry and token), against the dense f16 peak"},
         "scan_key_bytes": scan_bytes, "reindex_bytes": reindex_bytes(wl, pn, n_vis)})
    print(json.dumps(result), flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="full_1m_b4",
                    choices=["full_1m_b4", "full_8k_b1", "group_128k_b8", "schedule_20l_b32", "cache_write_1m",
                             "prefill_256t_1m"])
    ap.add_argument("--copies", type=int, default=4, help="rotated cache copies (> 512 MB touched)")
    ap.add_argument("--steps-per-graph", type=int, default=8,
                    help="consecutive layer steps per replayed graph (cache copy = step mod copies)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kidx-format", choices=["e4m3", "mxfp4"], default="e4m3",
                    help="indexer-key format: E4M3 (128 B per entry) or the pages' MXFP4 (68 B per entry, "
                         "random synthetic codes and scales)")
    ap.add_argument("--score-path", choices=["fast", "general-q", "general-k"], default="fast",
                    help="indexer inputs of the default workload: N(0,1) (the f16 two-limb path), queries "
                         "N(0, 64^2) (every row on the int8 general path) or keys N(0, 4^2) (every chunk on it)")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of HIP-graph replays")
    ap.add_argument("--counters", action="store_true",
                    help="only launch the counter-calibration sequence (for rocprofv3 --pmc runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this path has no multi-GPU leg (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2
    if args.counters:
        return counters_driver(args)
    if args.workload == "schedule_20l_b32":
        return bench_schedule(args)
    if args.workload == "group_128k_b8":
        return bench_group(args)
    if args.workload == "cache_write_1m":
        return bench_cache_write(args)
    if args.workload == "prefill_256t_1m":
        return bench_prefill(args)
    return bench_layer(args)


if __name__ == "__main__":
    sys.exit(main())
