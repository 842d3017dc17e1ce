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
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "score_full_1m_b4_hbm_traffic.md")
INDEX_SRC = os.path.join(ROOT, "compressed_sparse_attention_mxfp4_amd", "csrc", "index.hip")


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

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.rt.hipEventCreate(ctypes.byref(e)) == 0
            evs.append(e)
        return evs

    def elapsed_ms(self, a, b):
        f = ctypes.c_float()
        st = self.rt.hipEventElapsedTime(ctypes.byref(f), a, b)
        return float(f.value) if st == 0 else float("nan")

    def destroy(self, evs):
        for e in evs:
            self.rt.hipEventDestroy(e)


def algorithmic_bytes(wl, key_bytes=128):
    """Bytes the method must move per layer step (inputs read + outputs written);
    key_bytes: bytes per indexer key (128 E4M3, 68 MXFP4)."""
    n = int(np.sum(wl.n_entries))
    B, T, H, HI, k = wl.B, wl.T, wl.H, wl.HI, wl.topk
    scan = n * key_bytes + B * T * HI * (128 + 4)           # indexer keys + queries + weights
    idx_out = B * T * (k + wl.pool_blocks + 1) * 4           # top-k, pool, count
    sel = min(k, int(wl.n_entries.min()))
    gather = B * T * sel * 288                               # selected FP4 entries
    swa = B * (127 + T) * 512                                 # FP8 window
    attn_io = B * T * H * 512 * 2 + B * T * H * 512 * 4      # q bf16 in, out fp32
    write = B * T * (1024 + 8 + 288)                         # new rows: bf16 in, slot, FP4 out
    return {"scan": scan, "step": scan + idx_out + gather + swa + attn_io + write}


def measured_traffic():
    """HBM bytes per score-scan launch from the committed counter summary
    (FETCH_SIZE and WRITE_SIZE scaled by a plain copy's readings), or None
    when the scan's source has changed since the counters were taken."""
    import hashlib
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = dict(line.split(": ", 1) for line in text.splitlines() if line.startswith(("traffic_bytes", "index_hip")))
    digest = hashlib.sha256(open(INDEX_SRC, "rb").read()).hexdigest()
    if fields.get("index_hip_sha256", "").strip() != digest:
        return None
    return int(fields["traffic_bytes_per_launch"])


def counters_driver(args):
    """Launch sequence for rocprofv3 counter runs: a plain 256 MiB device copy
    (calibrates FETCH_SIZE / WRITE_SIZE), then 3 times each: the Full indexer
    of the workload, the same over MXFP4 indexer keys, the cache write of all
    of the workload's rows (1,048,576 at 1M context), the fused RoPE + cache
    writes of those rows, the compressor forming that many entries at 4:1
    and the sparse attention over the indexer's top-k."""
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
        topk = csa2.index_full(q, w, kidx, pt, ne, wl.max_n, wl.topk, wl.pool_blocks, ws=ws)[0]
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


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="full_1m_b4")
    ap.add_argument("--copies", type=int, default=4, help="rotated cache copies (> 512 MB touched)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kidx-format", choices=["e4m3", "mxfp4"], default="e4m3",
                    help="indexer-key format: E4M3 (128 B per entry) or the pages' MXFP4 (68 B per entry, "
                         "random synthetic codes and scales)")
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
    import torch
    import compressed_sparse_attention_mxfp4_amd as csa2
    from compressed_sparse_attention_mxfp4_amd import synth
    if not os.path.exists(csa2.LIB_PATH):
        from compressed_sparse_attention_mxfp4_amd import build
        build.build()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    csa2.load()
    dev = torch.device("cuda:0")

    t0 = time.perf_counter()
    wl = synth.workload(args.workload)
    L = wl.layers[0]
    log(f"workload {args.workload} generated in {time.perf_counter() - t0:.1f} s")

    def up(a, dtype=None):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(dtype) if dtype is not None else t).to(dev)

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
    # the step's own cache write: each sequence's newest entry, re-written from its bf16 row
    last = np.cumsum(wl.n_entries) - 1
    new_rows = kv_src[torch.from_numpy(last).to(dev)].contiguous()
    new_slots = slots[torch.from_numpy(last).to(dev)].contiguous()
    del kv_src
    B, T, H = wl.B, wl.T, wl.H
    out_topk = torch.empty((B, T, wl.topk), dtype=torch.int32, device=dev)
    out_pool = torch.empty((B, T, wl.pool_blocks), dtype=torch.int32, device=dev)
    out_pool_n = torch.empty((B, T), dtype=torch.int32, device=dev)
    out = torch.empty((B, T, H, 512), dtype=torch.float32, device=dev)
    ws_i, ws_a = csa2.Workspace(), csa2.Workspace()
    stream = torch.cuda.current_stream()

    def step(i, strm):
        c = i % args.copies
        # the cache write rides in the indexer's launches (csa2_index_full[_mxfp4]_write); it
        # lands before the attention, which reads the new entries
        csa2.index_full(q_idx, w, kidx[c], pt, ne, wl.max_n, wl.topk, wl.pool_blocks, out_topk=out_topk,
                        out_pool=out_pool, out_pool_n=out_pool_n, ws=ws_i, stream=strm, mxfp4=mx,
                        write=(new_rows, new_slots, kvp[c]))
        csa2.sparse_attn(q, wl.sm_scale, kvp[c], pt, ne, out_topk, swa, out=out, ws=ws_a, stream=strm)

    for i in range(args.warmup):
        step(i, stream)
    torch.cuda.synchronize()
    ev = HipEvents()
    ev.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    K = args.steps

    # ---- pass 1: per-kernel durations (eager launches, event pair around each launch)
    kernels = {"score_full": csa2.K_SCORE_FULL, "select_full": csa2.K_SELECT_FULL,
               "attn_split": csa2.K_ATTN_SPLIT, "attn_combine": csa2.K_ATTN_COMBINE}
    pairs = {name: (ev.create(K), ev.create(K)) for name in kernels}
    torch.cuda.synchronize()
    for i in range(K):
        for name, kid in kernels.items():
            csa2.lib().csa2_time_kernel(kid, pairs[name][0][i], pairs[name][1][i])
        step(args.warmup + i, stream)
    torch.cuda.synchronize()
    for kid in kernels.values():
        csa2.lib().csa2_time_kernel(kid, None, None)
    kern_us = {name: 1000.0 * float(np.mean([ev.elapsed_ms(a, b) for a, b in zip(*pairs[name])]))
               for name in kernels}
    for a, b in pairs.values():
        ev.destroy(a)
        ev.destroy(b)
    eager_ref = out_topk.clone(), out.clone()

    # ---- pass 2: whole steps, timed with one event pair around K steps
    graphs = None
    if not args.eager:
        # one captured step per cache copy; the library makes no allocation or memset
        graphs = []
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for c in range(args.copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    step(c, torch.cuda.current_stream())
                graphs.append(g)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        # a replay reproduces the eager step (same copy as the last eager step)
        last = (args.warmup + K - 1) % args.copies
        graphs[last].replay()
        torch.cuda.synchronize()
        assert torch.equal(out_topk, eager_ref[0]) and torch.equal(out, eager_ref[1]), \
            "graph replay differs from the eager step"
        for i in range(args.warmup):
            graphs[i % args.copies].replay()
        torch.cuda.synchronize()

    def run_step(i):
        if graphs is not None:
            graphs[i % args.copies].replay()
        else:
            step(i, stream)

    whole = ev.create(2)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev.rt.hipEventRecord(whole[0], ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    for i in range(K):
        run_step(i)
    ev.rt.hipEventRecord(whole[1], ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = ev.elapsed_ms(whole[0], whole[1])

    ms_per_step = total_ms / K
    value = 1000.0 / ms_per_step
    nbytes = algorithmic_bytes(wl, 68 if mx else 128)
    scan_gbs = nbytes["scan"] / (kern_us["score_full"] * 1e-6) / 1e9
    step_gbs = nbytes["step"] / (ms_per_step * 1e-3) / 1e9
    log(f"{K} steps ({'eager' if graphs is None else 'graph replay'}): {ms_per_step * 1000:.1f} us/step "
        f"(wall {wall / K * 1e6:.1f} us/step); kernels us: "
        + ", ".join(f"{k}={v:.1f}" for k, v in kern_us.items()))

    result = {
        "metric": "CSA2 decode layer-steps/s at 1M ctx; achieved HBM TB/s and % of peak",
        "value": round(value, 2),
        "unit": "layer-steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8/fp4 storage; f16-MFMA exact scores (int8-MFMA general path); f16-MFMA attention; fp32 softmax",
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": B, "query_tokens": T,
                   "context_tokens": int(wl.max_n) * 4, "entries_per_seq": int(wl.max_n),
                   "indexer_heads": wl.HI, "heads": H, "topk": wl.topk, "pool_blocks": wl.pool_blocks,
                   "indexer_key_format": args.kidx_format, "cache_copies_rotated": args.copies,
                   "launch": "eager" if graphs is None else "hip_graph_replay"},
        "hbm_tb_s": round(step_gbs / 1000.0, 3),
        "hbm_frac_of_peak": round(step_gbs / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": nbytes["step"],
        "kernel_avg_us": {k: round(v, 2) for k, v in kern_us.items()},
        "roofline": {"kernel": "score_kernel (Full-mode exact score scan)", "bound": "hbm",
                     "achieved": round(scan_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(scan_gbs / HBM_PEAK_GBS, 4), "traffic": None if mx else measured_traffic(),
                     "algorithmic_bytes_per_launch": nbytes["scan"]},
    }
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        result["cpu_baseline"] = cpu_baseline(wl, kidx_mx=kidx_mx)
        log(f"cpu baseline in {time.perf_counter() - t0:.1f} s")
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
