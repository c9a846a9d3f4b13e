#!/usr/bin/env python3
"""Benchmark of the paged varlen attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass of the whole path over one batch: the batch's new K/V
rows stored into the paged cache, then attention over it.  For the decode
batch that is one attn_decode_append_paged call (store and attention in one
launch; the two-call form, kv_store_paged then attn_varlen_paged, is timed
beside it); for prefill it is the two calls.  The headline workload is the
paged decode batch (64 sequences x 1 query row, contexts uniform in
[128, 2048], 32 query / 8 KV heads, head dim 64, bf16, 16-token pages,
shuffled blocks); its metric is K+V bytes read per second.  The causal prefill
batch (16 x 512 tokens, 32/8 heads, head dim 128, bf16) is measured the same
way and reported under "prefill" in attention TFLOP/s.

Timing follows the device-event method of Transformer 추론 커널 (3/10), §26:
warm-up launches, then K back-to-back steps between two events on the stream;
the steps are replayed from captured HIP graphs, so the host's time to issue
each call does not enter the figure (--eager times plain launches instead).
Each step uses the next of R replicas (separate device copies of the same
batch) so that the 256 MB Infinity Cache cannot hold the working set.
Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def _src_sha(names) -> str:
    """Hash of a kernel's source files together with the shared headers and the
    planner that sets its launch shape."""
    h = hashlib.sha256()
    for f in (*names, "kvs_device.hpp", "kvs_internal.hpp", "api.hip"):
        h.update(open(os.path.join(ROOT, "attention_kv_store_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


# kernel symbol (as rocprofv3 names it) and source file of each timed workload
# (a batch of several sequences with T != B runs as one mixed launch, whose
# grid here holds only prefill items; a single prompt runs in the prefill kernel)
MIXED_SRC = ("mixed.hip", "prefill_impl.hpp", "decode_impl.hpp")
COUNTED = {
    "paged_decode_bf16": ("kvs::decode_kernel<64, true, true, false, false, false, false>", ("decode.hip", "decode_impl.hpp")),
    "causal_prefill_bf16": ("kvs::mixed_kernel<128, false, 4>", MIXED_SRC),
    "extend_prefill_bf16": ("kvs::mixed_kernel<128, false, 4>", MIXED_SRC),
    "long_prefill_bf16": ("kvs::prefill_kernel<128, true, 8, false, false, false>", ("prefill.hip", "prefill_impl.hpp")),
}


READ_COUNTERS = ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_32B_sum", "TCC_BUBBLE_sum", "TCC_EA0_RDREQ_DRAM_sum")
WRITE_COUNTERS = ("TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_64B_sum", "TCC_EA0_WRREQ_DRAM_sum")


def summarize_counters(specs, command: str) -> None:
    """Turn rocprofv3 --pmc runs of this script into HBM bytes per launch.
    Each spec is WORKLOAD=READ_CSV,WRITE_CSV: two runs of one command (the
    workload's kernel among its dispatches), the first counting the L2's read
    requests to the memory side (READ_COUNTERS: all, 32-byte, 128-byte, and
    those bound for DRAM), the second its write requests (WRITE_COUNTERS: all,
    64-byte, bound for DRAM).

    Bytes are the request counts times their sizes (128 B for TCC_BUBBLE, 32 B
    for the 32-byte ones, 64 B for the rest; writes 64 B or 32 B).  The same
    sums are taken for a copy of known size -- the kv_store_paged launch that
    fills a decode replica's pool, 2 * sum(Lk) * Hkv * D * 2 bytes of K+V read
    and written plus the int32 slots read -- and the ratio of the known to the
    counted bytes is recorded as a check on those sizes; the per-launch
    figures are then given both as counted and scaled by that ratio."""
    import csv

    from workloads import kv_bytes, paged_decode_bf16

    def load(path, names):
        rows = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] in names:
                d = rows.setdefault(int(r["Dispatch_Id"]), {"kernel": r["Kernel_Name"]})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        return rows

    runs = {}
    for spec in specs:
        wl, _, files = spec.partition("=")
        rpath, _, wpath = files.partition(",")
        if wl not in COUNTED or not rpath or not wpath:
            raise SystemExit(f"bad spec {spec!r}: WORKLOAD=READ_CSV,WRITE_CSV with WORKLOAD one of {sorted(COUNTED)}")
        if (rpath, wpath) not in runs:
            runs[(rpath, wpath)] = (load(rpath, READ_COUNTERS), load(wpath, WRITE_COUNTERS))
        runs[wl] = runs[(rpath, wpath)]

    def rbytes(c):
        req, r32, r128 = c["TCC_EA0_RDREQ_sum"], c["TCC_EA0_RDREQ_32B_sum"], c["TCC_BUBBLE_sum"]
        return 128 * r128 + 32 * r32 + 64 * (req - r128 - r32)

    def wbytes(c):
        req, w64 = c["TCC_EA0_WRREQ_sum"], c["TCC_EA0_WRREQ_64B_sum"]
        return 64 * w64 + 32 * (req - w64)

    dec = paged_decode_bf16()
    copy_bytes = kv_bytes(dec)                       # K+V rows written (and read)
    slot_bytes = 4 * int(dec.k_lens.sum())
    # the copy: every run's pool-filling kv_store_paged launches
    cal = []
    for key, (rd, wr) in runs.items():
        if isinstance(key, tuple):
            cal += [(rd[i], wr[i]) for i, c in wr.items() if "kv_store_kernel" in c["kernel"] and i in rd
                    and abs(wbytes(c) - copy_bytes) < 0.05 * copy_bytes]
    if not cal:
        raise SystemExit("no full-pool kv_store_paged dispatch found for calibration")
    cr = sum(rbytes(r) for r, _ in cal) / len(cal)
    cw = sum(wbytes(w) for _, w in cal) / len(cal)
    read_factor = (copy_bytes + slot_bytes) / cr
    write_factor = copy_bytes / cw

    def mean(rows, ids, key):
        return sum(rows[i][key] for i in ids) / len(ids)

    def cal_mean(key):
        return sum(r[key] for r, _ in cal) / len(cal)

    out = {"_calibration": {
        "copy": f"kv_store_paged of all {int(dec.k_lens.sum())} context rows of paged_decode_bf16",
        "copy_read_bytes": copy_bytes + slot_bytes, "copy_write_bytes": copy_bytes,
        "counted_read_bytes": round(cr), "counted_write_bytes": round(cw),
        "read_requests": round(cal_mean("TCC_EA0_RDREQ_sum")),
        "read_requests_32B": round(cal_mean("TCC_EA0_RDREQ_32B_sum")),
        "read_requests_128B": round(cal_mean("TCC_BUBBLE_sum")),
        "known_over_counted_read": round(read_factor, 5), "known_over_counted_write": round(write_factor, 5),
        "dispatches": len(cal), "command": command}}
    for wl, (sym, src) in COUNTED.items():
        if wl not in runs:
            continue
        rd, wr = runs[wl]
        ids = [i for i, c in rd.items() if sym in c["kernel"] and i in wr]
        if not ids:
            raise SystemExit(f"{wl}: no dispatch of {sym} in its runs")
        req = mean(rd, ids, "TCC_EA0_RDREQ_sum")
        r_counted = sum(rbytes(rd[i]) for i in ids) / len(ids)
        w_counted = sum(wbytes(wr[i]) for i in ids) / len(ids)
        out[wl] = {"kernel": sym, "kernel_src_sha": _src_sha(src), "dispatches": len(ids),
                   "read_requests": round(req),
                   "read_requests_32B": round(mean(rd, ids, "TCC_EA0_RDREQ_32B_sum")),
                   "read_requests_128B": round(mean(rd, ids, "TCC_BUBBLE_sum")),
                   "read_requests_to_dram_frac": round(mean(rd, ids, "TCC_EA0_RDREQ_DRAM_sum") / max(req, 1.0), 4),
                   "write_requests": round(mean(wr, ids, "TCC_EA0_WRREQ_sum")),
                   "write_requests_64B": round(mean(wr, ids, "TCC_EA0_WRREQ_64B_sum")),
                   "read_bytes_counted": round(r_counted), "write_bytes_counted": round(w_counted),
                   "read_bytes_per_launch": round(r_counted * read_factor),
                   "write_bytes_per_launch": round(w_counted * write_factor),
                   "hbm_bytes_per_launch": round(r_counted * read_factor + w_counted * write_factor)}
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")
    log(json.dumps(out, indent=1))


def _traffic(kernel_src, workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, or None when
    the kernel source changed since they were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))[workload]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("kernel_src_sha") != _src_sha(kernel_src):
        return None
    return rec.get("hbm_bytes_per_launch")


class Workload:
    """R device replicas of one host batch, plus the step function."""

    def __init__(self, batch, replicas: int, decode_tail: int = 0):
        import torch
        from workloads.device import to_device

        self.batch = batch
        self.reps = []
        rows = batch.new_token_rows()
        dt = torch.bfloat16 if batch.dtype == "bf16" else torch.float32
        for _ in range(replicas):
            db = to_device(batch)                      # pool filled by kv_store_paged
            kn = torch.from_numpy(batch.k_tokens[rows]).to(dt).cuda()
            vn = torch.from_numpy(batch.v_tokens[rows]).to(dt).cuda()
            sl = torch.from_numpy(batch.slots[rows]).cuda()
            out = torch.empty_like(db.q)
            lse = torch.empty(db.q.shape[0], db.q.shape[1], dtype=torch.float32, device="cuda")
            self.reps.append((db, kn, vn, sl, out, lse))
        import attention_kv_store_amd as kvs
        self.kvs = kvs
        db = self.reps[0][0]
        self.decode_tail = int(decode_tail)
        need = kvs.workspace_size(db.q, db.k_cache, db.block_table, decode_tail=self.decode_tail)
        self.ws = [torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda") for _ in range(replicas)]
        torch.cuda.synchronize()

    def store(self, i):
        db, kn, vn, sl, _, _ = self.reps[i % len(self.reps)]
        self.kvs.kv_store_paged(kn, vn, sl, db.k_cache, db.v_cache)

    def attend(self, i):
        r = i % len(self.reps)
        db, _, _, _, out, lse = self.reps[r]
        self.kvs.attn_varlen_paged(db.q, db.k_cache, db.v_cache, db.block_table, db.cu_seqlens_q,
                                   db.seqlens_k, db.scale, db.causal, out=out, lse=lse, workspace=self.ws[r],
                                   window=self.batch.window, decode_tail=self.decode_tail)

    def append_attend(self, i):
        r = i % len(self.reps)
        db, kn, vn, _, out, lse = self.reps[r]
        self.kvs.attn_decode_append_paged(db.q, kn, vn, db.k_cache, db.v_cache, db.block_table, db.seqlens_k,
                                          db.scale, out=out, lse=lse, workspace=self.ws[r],
                                          window=self.batch.window)


def _graph_len(steps: int, cap: int = 100) -> int:
    """Steps per captured graph: the largest divisor of ``steps`` up to ``cap``,
    so that whole replays time exactly ``steps`` steps."""
    return max(d for d in range(1, min(steps, cap) + 1) if steps % d == 0)


def time_steps(w: Workload, steps: int, warmup: int, fused: bool = False, eager: bool = False):
    """Time exactly ``steps`` steps on one stream.

    The steps are captured into a HIP graph (G steps per graph, G dividing
    ``steps``) and the graph is replayed steps / G times between two events, so
    the figure is the device's time per step, not the host's time to issue it;
    a serving loop issues decode steps the same way ("장부가 커널 인자로 바뀌는
    지점과 CUDA graph").  A second graph holding only the attention launches of
    the same steps gives that launch's average duration.  With ``fused`` a step
    is the one attn_decode_append_paged launch, and the two figures coincide.

    With ``eager`` the steps are plain launches instead, with events around
    each attention call (host issue time included where it exceeds the
    device's).

    Returns (ms per step, ms per attention launch, wall seconds, stats) where
    stats holds the median and p95 over the graph replays of the per-step
    time (None for eager timing)."""
    import torch

    store = (lambda i: None) if fused else w.store
    attend = w.append_attend if fused else w.attend
    for i in range(warmup):
        store(i)
        attend(i)
    torch.cuda.synchronize()
    if eager:
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        start.record()
        for i in range(steps):
            store(i)
            ev[i][0].record()
            attend(i)
            ev[i][1].record()
        end.record()
        torch.cuda.synchronize()
        return (start.elapsed_time(end) / steps, sum(a.elapsed_time(b) for a, b in ev) / steps,
                time.perf_counter() - t0, None)
    G = _graph_len(steps)

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(G):
                fn(i)
        return g

    def run(g):
        for _ in range(2):                      # replay warm-up
            g.replay()
        torch.cuda.synchronize()
        nrep = steps // G
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(nrep + 1)]
        t0 = time.perf_counter()
        ev[0].record()
        for r in range(nrep):
            g.replay()
            ev[r + 1].record()
        torch.cuda.synchronize()
        per = sorted(ev[r].elapsed_time(ev[r + 1]) / G for r in range(nrep))
        stats = {"replays": nrep, "steps_per_replay": G, "median_ms_per_step": round(per[nrep // 2], 6),
                 "p95_ms_per_step": round(per[min(nrep - 1, int(0.95 * nrep))], 6)}
        return ev[0].elapsed_time(ev[nrep]) / steps, time.perf_counter() - t0, stats

    g_step = capture(lambda i: (store(i), attend(i)))
    ms_step, wall, stats = run(g_step)
    if fused:
        attn_ms = ms_step
    else:
        g_attn = capture(attend)
        attn_ms, _, astats = run(g_attn)
        stats["attention_median_ms"] = astats["median_ms_per_step"]
        del g_attn
    del g_step
    return ms_step, attn_ms, wall, stats


def runner_replays(dec, args):
    """Replay time of DecodeGraphRunner's 64-row bucket for 64 real rows and
    for 50 real rows padded with 14 dummy rows (one key each)."""
    import torch

    from attention_kv_store_amd.graph_runner import DecodeGraphRunner
    from workloads.device import to_device

    db = to_device(dec)
    rows = dec.new_token_rows()
    kn = torch.from_numpy(dec.k_tokens[rows]).to(torch.bfloat16).cuda()
    vn = torch.from_numpy(dec.v_tokens[rows]).to(torch.bfloat16).cuda()
    runner = DecodeGraphRunner(db.k_cache, db.v_cache, dec.poison_block, [16, 32, 64], dec.MB, Hq=dec.Hq,
                               scale=dec.scale)
    res = {}
    for B in (64, 50):
        runner.step(db.q[:B], kn[:B], vn[:B], db.block_table[:B], db.seqlens_k[:B])
        g = runner.graphs[runner.bucket_for(B)]
        n = max(50, args.steps // 20)
        for _ in range(5):
            g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        res[f"rows_{B}_bucket_64_us"] = round(e0.elapsed_time(e1) / n * 1e3, 3)
    res["note"] = "one replica (cache-resident between replays); the headline rotates 4 replicas"
    del runner, db
    torch.cuda.empty_cache()
    return res


def _q8_calls(fmt):
    """(cache dtype, quantizing store, attention, fused decode step) of the FP8
    (E4M3) or INT8 cache."""
    import torch
    import attention_kv_store_amd as kvs
    if fmt == "int8":
        return torch.int8, kvs.kv_store_paged_int8, kvs.attn_varlen_paged_int8, kvs.attn_decode_append_paged_int8
    return torch.uint8, kvs.kv_store_paged_fp8, kvs.attn_varlen_paged_fp8, kvs.attn_decode_append_paged_fp8


def fp8_line(batch, args, n=100, fmt="fp8"):
    """A workload over an FP8 (E4M3) or INT8 cache: every key row quantized by
    kv_store_paged_fp8 / _int8 (one scale per row and KV head), then
    attn_varlen_paged_fp8 / _int8 timed from graph replays over 4 replicas.
    Bytes read per launch: the codes of every visible key row of K and V plus
    their fp32 scales."""
    import torch
    import attention_kv_store_amd as kvs
    from workloads import attention_flops

    cdt, store, attn, _ = _q8_calls(fmt)
    rows = batch.store_rows()
    reps = []
    for r in range(4):
        kc = torch.zeros(batch.pool_shape(), dtype=cdt, device="cuda")
        vc = torch.zeros_like(kc)
        ks = torch.zeros(batch.num_blocks, batch.Hkv, 16, dtype=torch.float32, device="cuda")
        vs = torch.zeros_like(ks)
        store(torch.from_numpy(batch.k_tokens[rows]).to(torch.bfloat16).cuda(),
              torch.from_numpy(batch.v_tokens[rows]).to(torch.bfloat16).cuda(),
              torch.from_numpy(batch.slots[rows]).cuda(), kc, vc, ks, vs)
        q = torch.from_numpy(batch.q).to(torch.bfloat16).cuda()
        meta = [torch.from_numpy(x).cuda() for x in (batch.block_table, batch.cu_seqlens_q, batch.k_lens)]
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device="cuda")
        ws = torch.zeros(max(kvs.workspace_size(q, kc, meta[0]), 1), dtype=torch.uint8, device="cuda")
        reps.append((q, kc, vc, ks, vs, meta, out, lse, ws))

    def call(i):
        q, kc, vc, ks, vs, meta, out, lse, ws = reps[i % 4]
        attn(q, kc, vc, ks, vs, *meta, batch.scale, batch.causal, out=out, lse=lse, workspace=ws)

    for i in range(8):
        call(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n):
            call(i)
    graph.replay()
    torch.cuda.synchronize()
    nrep = max(2, args.steps // (4 * n)) if batch.T != batch.B else max(2, args.steps // n)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(nrep):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / (nrep * n) * 1e3
    nkeys = int(batch.k_lens.sum())
    read = 2 * nkeys * batch.Hkv * (batch.D + 4)        # codes and scales of K and V
    res = {"workload": f"{batch.name} with an {'INT8' if fmt == 'int8' else 'FP8 (E4M3)'} cache", "avg_launch_us": round(us, 3),
           "kv_bytes_per_launch": read, "kv_GBs": round(read / (us * 1e-6) / 1e9, 1),
           "TFLOPs": round(attention_flops(batch) / (us * 1e-6) / 1e12, 1), "dispatch": kvs.last_dispatch()}
    del graph, reps
    torch.cuda.empty_cache()
    return res


def context_sweep(args):
    """Decode over 64 sequences at contexts 512, 4096 and 16384 (all of one
    length), 32 / 8 heads, D 128, bf16 -- the decode microbenchmark shape the
    pages' manifest lists.  Pools filled on the device (torch.randn), block
    tables random permutations; replicas so that the rotation exceeds the
    256 MB Infinity Cache.  Timed from graph replays of attn_varlen_paged."""
    import torch
    import attention_kv_store_amd as kvs

    B, Hq, Hkv, D = 64, 32, 8, 128
    res = {}
    for ctx in (512, 4096, 16384):
        nblk = B * ctx // 16
        kv_bytes = 2 * B * ctx * Hkv * D * 2
        R = max(1, -(-512 * 2**20 // kv_bytes))
        reps = []
        g = torch.Generator(device="cuda").manual_seed(ctx)
        for r in range(R):
            kc = torch.randn(nblk + 1, 16, Hkv, D, device="cuda", generator=g).to(torch.bfloat16)
            vc = torch.randn(nblk + 1, 16, Hkv, D, device="cuda", generator=g).to(torch.bfloat16)
            table = torch.randperm(nblk, device="cuda", generator=g).to(torch.int32).view(B, ctx // 16).contiguous()
            q = torch.randn(B, Hq, D, device="cuda", generator=g).to(torch.bfloat16)
            lens = torch.full((B,), ctx, dtype=torch.int32, device="cuda")
            cu = torch.arange(B + 1, dtype=torch.int32, device="cuda")
            ws = torch.zeros(max(kvs.workspace_size(q, kc, table), 1), dtype=torch.uint8, device="cuda")
            reps.append((q, kc, vc, table, cu, lens, torch.empty_like(q),
                         torch.empty(B, Hq, dtype=torch.float32, device="cuda"), ws))

        def call(i):
            q, kc, vc, table, cu, lens, out, lse, ws = reps[i % R]
            kvs.attn_varlen_paged(q, kc, vc, table, cu, lens, D ** -0.5, True, out=out, lse=lse, workspace=ws)

        for i in range(4):
            call(i)
        torch.cuda.synchronize()
        n = 40
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(n):
                call(i)
        graph.replay()
        torch.cuda.synchronize()
        nrep = 5
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(nrep):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / (nrep * n) * 1e3
        res[f"context_{ctx}"] = {"us": round(us, 2), "kv_bytes": kv_bytes, "replicas": R,
                                 "GBs": round(kv_bytes / (us * 1e-6) / 1e9, 1),
                                 "frac": round(kv_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                                 "dispatch": kvs.last_dispatch()}
        del graph, reps
        torch.cuda.empty_cache()
    return res


def rope_decode_line(dec, args):
    """A decode step of a RoPE model on the decode workload: the fused step with
    RoPE inside (one launch) against kv_store_rope_paged + attn_varlen_paged
    (two launches), graph replays over 4 replicas."""
    import torch
    import attention_kv_store_amd as kvs

    w = Workload(dec, 4)
    rows = dec.new_token_rows()
    pos = torch.from_numpy((dec.k_lens - 1).astype("int32")).cuda()
    res = {}

    def fused(i):
        db, kn, vn, _, out, lse = w.reps[i % 4]
        kvs.attn_decode_append_paged(db.q, kn, vn, db.k_cache, db.v_cache, db.block_table, db.seqlens_k, db.scale,
                                     out=out, lse=lse, workspace=w.ws[i % 4], rope={"style": "neox"})

    def two(i):
        db, kn, vn, sl, out, lse = w.reps[i % 4]
        kvs.kv_store_rope_paged(db.q, kn, vn, pos, sl, db.k_cache, db.v_cache)
        kvs.attn_varlen_paged(db.q, db.k_cache, db.v_cache, db.block_table, db.cu_seqlens_q, db.seqlens_k, db.scale,
                              True, out=out, lse=lse, workspace=w.ws[i % 4])

    for name, fn in (("fused_one_launch", fused), ("rope_store_then_attention", two)):
        for i in range(8):
            fn(i)
        torch.cuda.synchronize()
        n = 100
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(n):
                fn(i)
        graph.replay()
        torch.cuda.synchronize()
        nrep = max(2, args.steps // n)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(nrep):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        res[name] = {"us_per_step": round(e0.elapsed_time(e1) / (nrep * n) * 1e3, 3), "dispatch": kvs.last_dispatch()}
        del graph
    del w
    torch.cuda.empty_cache()
    return res


def fp8_step_line(dec, args, fmt="fp8"):
    """A decode step over an FP8 or INT8 cache on the decode workload: the
    fused step (attn_decode_append_paged_fp8 / _int8, one launch) against the
    quantizing store of the 64 new rows + the attention (two launches)."""
    import torch
    import attention_kv_store_amd as kvs

    cdt, store, attn, fused_call = _q8_calls(fmt)
    rows, new = dec.store_rows(), dec.new_token_rows()
    reps = []
    for r in range(4):
        kc = torch.zeros(dec.pool_shape(), dtype=cdt, device="cuda")
        vc = torch.zeros_like(kc)
        ks = torch.zeros(dec.num_blocks, dec.Hkv, 16, dtype=torch.float32, device="cuda")
        vs = torch.zeros_like(ks)
        store(torch.from_numpy(dec.k_tokens[rows]).to(torch.bfloat16).cuda(),
              torch.from_numpy(dec.v_tokens[rows]).to(torch.bfloat16).cuda(),
              torch.from_numpy(dec.slots[rows]).cuda(), kc, vc, ks, vs)
        q = torch.from_numpy(dec.q).to(torch.bfloat16).cuda()
        kn = torch.from_numpy(dec.k_tokens[new]).to(torch.bfloat16).cuda()
        vn = torch.from_numpy(dec.v_tokens[new]).to(torch.bfloat16).cuda()
        sl = torch.from_numpy(dec.slots[new]).cuda()
        meta = [torch.from_numpy(x).cuda() for x in (dec.block_table, dec.cu_seqlens_q, dec.k_lens)]
        ws = torch.zeros(max(kvs.workspace_size(q, kc, meta[0]), 1), dtype=torch.uint8, device="cuda")
        reps.append((q, kn, vn, sl, kc, vc, ks, vs, meta, torch.empty_like(q),
                     torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device="cuda"), ws))

    def fused(i):
        q, kn, vn, sl, kc, vc, ks, vs, meta, out, lse, ws = reps[i % 4]
        fused_call(q, kn, vn, kc, vc, ks, vs, meta[0], meta[2], dec.scale, out=out, lse=lse, workspace=ws)

    def two(i):
        q, kn, vn, sl, kc, vc, ks, vs, meta, out, lse, ws = reps[i % 4]
        store(kn, vn, sl, kc, vc, ks, vs)
        attn(q, kc, vc, ks, vs, *meta, dec.scale, True, out=out, lse=lse, workspace=ws)

    res = {}
    for name, fn in (("fused_one_launch", fused), ("store_then_attention", two)):
        for i in range(8):
            fn(i)
        torch.cuda.synchronize()
        n = 100
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(n):
                fn(i)
        graph.replay()
        torch.cuda.synchronize()
        nrep = max(2, args.steps // n)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(nrep):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        res[name] = {"us_per_step": round(e0.elapsed_time(e1) / (nrep * n) * 1e3, 3), "dispatch": kvs.last_dispatch()}
        del graph
    del reps
    torch.cuda.empty_cache()
    return res


def rope_store_line(args):
    """kv_store_rope_paged at the causal prefill workload's shape (16 x 512 new
    rows, 32 / 8 heads, D 128) and the decode workload's (64 rows, 32 / 8 heads,
    D 64), bf16, timed from graph replays over 4 replicas.  Bytes moved: Q read
    and written, K and V rows read and written, positions and slots read."""
    import torch
    import attention_kv_store_amd as kvs

    res = {}
    for name, T, Hq, Hkv, D in (("prefill_rows", 8192, 32, 8, 128), ("decode_rows", 64, 32, 8, 64)):
        reps = []
        NB = (T + 15) // 16 + 1
        for r in range(4):
            g = torch.Generator(device="cuda").manual_seed(r)
            q = torch.randn(T, Hq, D, device="cuda", generator=g).to(torch.bfloat16)
            kn = torch.randn(T, Hkv, D, device="cuda", generator=g).to(torch.bfloat16)
            vn = torch.randn(T, Hkv, D, device="cuda", generator=g).to(torch.bfloat16)
            pos = torch.arange(T, dtype=torch.int32, device="cuda") * 7
            slots = torch.randperm(NB * 16, device="cuda", generator=g)[:T].to(torch.int32)
            kc = torch.zeros(NB, 16, Hkv, D, dtype=torch.bfloat16, device="cuda")
            reps.append((q, kn, vn, pos, slots, kc, torch.zeros_like(kc)))

        def call(i):
            q, kn, vn, pos, slots, kc, vc = reps[i % 4]
            kvs.kv_store_rope_paged(q, kn, vn, pos, slots, kc, vc)

        for i in range(8):
            call(i)
        torch.cuda.synchronize()
        n = 100
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(n):
                call(i)
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nrep = max(2, args.steps // (4 * n))
        e0.record()
        for _ in range(nrep):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / (nrep * n) * 1e3
        moved = 2 * 2 * T * D * (Hq + 2 * Hkv) + 8 * T
        res[name] = {"rows": T, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D, "us": round(us, 3),
                     "bytes": moved, "GBs": round(moved / (us * 1e-6) / 1e9, 1),
                     "dispatch": kvs.last_dispatch()}
        del graph, reps
        torch.cuda.empty_cache()
    return res


def measure_peaks():
    """Rates this GPU sustains, to set beside the published peaks: a 1 GiB
    device-to-device copy (bytes read + written per second) and a bf16 MFMA
    loop with no memory traffic (kvs_mfma_peak_launch)."""
    import torch

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e-3

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    t_copy = timed(lambda: b.copy_(a), 10)
    copy_gbs = 2 * n / t_copy / 1e9
    del a, b
    # the calibration kernel lives in its own library (include/kvstore_calib.h)
    import ctypes
    calib = ctypes.CDLL(os.path.join(ROOT, "attention_kv_store_amd", "libkvstore_calib.so"))
    calib.kvs_mfma_peak_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_void_p]
    calib.kvs_mfma_peak_launch.restype = ctypes.c_int
    src = torch.randn(256, device="cuda").to(torch.bfloat16)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    wgs, iters = 8 * cus, 2048
    dst = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def mfma():
        st = calib.kvs_mfma_peak_launch(src.data_ptr(), dst.data_ptr(), wgs, iters, stream)
        if st != 0:
            raise RuntimeError(f"kvs_mfma_peak_launch failed with status {st}")

    t_mfma = timed(mfma, 5)
    flops = wgs * 4 * 4 * iters * 32768
    return {"copy_GBs": round(copy_gbs, 1), "bf16_mfma_TFLOPs": round(flops / t_mfma / 1e12, 1),
            "how": "1 GiB device copy (read + write bytes); bf16 32x32x16 MFMA loop, "
                   f"{wgs} workgroups x 4 waves x 4 chains x {iters} MFMAs, no memory traffic"}


def _git_head():
    """The checked-out commit, read from .git without running git (None where
    the tree travels without its history)."""
    try:
        with open(os.path.join(ROOT, ".git", "HEAD")) as fh:
            head = fh.read().strip()
        if head.startswith("ref: "):
            ref = head[5:]
            path = os.path.join(ROOT, ".git", ref)
            if os.path.exists(path):
                with open(path) as fh:
                    return fh.read().strip()[:7]
            with open(os.path.join(ROOT, ".git", "packed-refs")) as fh:
                return next((l.split()[0][:7] for l in fh if l.rstrip().endswith(" " + ref)), None)
        return head[:7] or None
    except (OSError, IndexError):
        return None


def _dpm_clocks():
    """The current DPM level of each clock domain the GPU's sysfs lists
    (pp_dpm_sclk, _mclk, _fclk, _socclk: the line marked '*'), or None.  Read
    from files: no program is started, which a process that has set up the
    GPU must not do."""
    out = {}
    try:
        cards = sorted(d for d in os.listdir("/sys/class/drm") if d.startswith("card") and d[4:].isdigit())
    except OSError:
        return None
    for card in cards:
        dev = os.path.join("/sys/class/drm", card, "device")
        for dom in ("sclk", "mclk", "fclk", "socclk"):
            try:
                with open(os.path.join(dev, "pp_dpm_" + dom)) as fh:
                    cur = next((l.split(":", 1)[1].replace("*", "").strip() for l in fh if "*" in l), None)
            except (OSError, IndexError):
                continue
            if cur:
                out.setdefault(card, {})[dom] = cur
    return out or None


def environment():
    import platform

    import torch

    env = {"device": torch.cuda.get_device_name(0), "torch": torch.__version__,
           "hip": getattr(torch.version, "hip", None), "host": platform.node(),
           "host_cpus": len(os.sched_getaffinity(0)), "git": _git_head()}
    # where the repository travels without its history: a hash of the sources
    # the library is built from
    h = hashlib.sha256()
    for d in (os.path.join(ROOT, "attention_kv_store_amd", "csrc"), os.path.join(ROOT, "include")):
        for f in sorted(os.listdir(d)):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    env["src_sha"] = h.hexdigest()[:16]
    try:
        with open("/proc/cpuinfo") as fh:
            env["host_cpu"] = next((l.split(":", 1)[1].strip() for l in fh if l.startswith("model name")), None)
    except OSError:
        env["host_cpu"] = None
    env["clocks"] = _dpm_clocks()
    return env


def _oracle_pool(batch):
    """The batch's paged pool as the oracle store builds it (NaN where no row
    is stored)."""
    import numpy as np

    from oracle import kv_store_oracle

    kc = np.full(batch.pool_shape(), np.nan)
    vc = np.full(batch.pool_shape(), np.nan)
    rows = batch.store_rows()
    return kv_store_oracle(batch.k_tokens[rows].astype(np.float64), batch.v_tokens[rows].astype(np.float64),
                           batch.slots[rows], kc, vc)


def _blas_threads() -> int:
    from threadpoolctl import threadpool_info

    info = threadpool_info()
    return int(max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1]))


def _parity(rows, ref_out, ref_lse, gpu_out, gpu_lse, tol, batch=None):
    """Error of the GPU's timed outputs against the oracle on `rows`: max-abs
    on out and lse (the pass criterion), and for out also the mean-abs error,
    the relative L2 error, the cosine similarity and, with `batch`, the
    max-abs error per band of visible keys (the long-context error growth
    check)."""
    import numpy as np

    ref = ref_out[rows]
    d = gpu_out - ref
    eo = float(np.max(np.abs(d)))
    el = float(np.max(np.abs(gpu_lse - ref_lse[rows])))
    finite = bool(np.isfinite(gpu_out).all() and np.isfinite(gpu_lse).all())
    res = {"rows": int(len(rows)), "max_abs_out": eo, "max_abs_lse": el, "tol": tol,
           "ok": bool(finite and eo <= tol and el <= tol),
           "mean_abs_out": float(np.mean(np.abs(d))),
           "rel_l2_out": float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)),
           "cosine_out": float(np.sum(gpu_out * ref) / max(np.linalg.norm(gpu_out) * np.linalg.norm(ref), 1e-300))}
    if batch is not None:
        vis = visible_keys(batch, np.asarray(rows))
        per_row = np.max(np.abs(d).reshape(len(rows), -1), axis=1)
        bands = {}
        for lo, hi in ((1, 256), (256, 1024), (1024, 4096), (4096, 16384), (16384, 1 << 31)):
            sel = (vis >= lo) & (vis < hi)
            if sel.any():
                bands[f"{lo}-{hi - 1 if hi < (1 << 31) else 'max'}"] = float(per_row[sel].max())
        res["max_abs_out_by_visible_keys"] = bands
    return res


def cpu_baseline(batch, gpu_out, gpu_lse, target_s: float = 10.0):
    """The oracle, untuned, on the same batch: repeated whole-batch calls until
    about target_s seconds of host time; K+V bytes / second.  Its result is
    also compared with the outputs of the GPU's last timed step."""
    import numpy as np

    from oracle import attention_oracle
    from workloads import kv_bytes

    kc, vc = _oracle_pool(batch)
    n, t = 0, 0.0
    while t < target_s:
        t0 = time.perf_counter()
        ro, rl = attention_oracle(batch.q, kc, vc, batch.block_table, batch.cu_seqlens_q, batch.k_lens,
                                  batch.scale, batch.causal, window=batch.window)
        t += time.perf_counter() - t0
        n += 1
    cores = _blas_threads()
    base = {"value": round(kv_bytes(batch) * n / t / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle",
            "sample": f"whole {batch.name} batch ({batch.T} rows, all heads), {n} calls in {t:.1f} s, "
                      f"numpy float64 with BLAS threads={cores}; {np.__version__}"}
    rows = np.arange(batch.T)
    return base, _parity(rows, ro, rl, gpu_out, gpu_lse, 2e-2, batch)


def visible_keys(batch, rows):
    """Keys each query row sees (causal bottom-right, optional window)."""
    import numpy as np

    seq = np.searchsorted(batch.cu_seqlens_q, rows, side="right") - 1
    i = rows - batch.cu_seqlens_q[seq]
    lq, lk = batch.q_lens[seq].astype(np.int64), batch.k_lens[seq].astype(np.int64)
    if not batch.causal:
        return lk
    pos = lk - lq + i
    vis = np.where(lq > 1, pos + 1, lk)
    if batch.window:
        vis = np.minimum(vis, batch.window)
    return vis


def cpu_baseline_prefill(batch, perm, kept, gpu_out, gpu_lse, target_s: float = 8.0):
    """The oracle, untuned, on a bounded sample of the workload's query rows
    (a seeded random order of all rows, its first n rows; n grown until one
    call takes at least target_s / 2 seconds), all heads.
    Value: the sample's algorithmic FLOPs (4 D per visible key and query head)
    per second.  The same rows are compared with the GPU's timed outputs
    (gpu_out / gpu_lse hold the sorted rows `kept`, a superset of the sample)."""
    import numpy as np

    from oracle import attention_oracle

    kc, vc = _oracle_pool(batch)
    per_row = 4.0 * batch.D * batch.Hq

    def run(n):
        rows = np.sort(perm[:n])
        t0 = time.perf_counter()
        ro, rl = attention_oracle(batch.q, kc, vc, batch.block_table, batch.cu_seqlens_q, batch.k_lens,
                                  batch.scale, batch.causal, window=batch.window, rows=rows)
        return time.perf_counter() - t0, rows, ro, rl

    # grow the sample until one call takes at least half of target_s (the
    # first calls are dominated by gathering the sequences' K / V)
    n = min(len(kept), 32)
    while True:
        t2, rows, ro, rl = run(n)
        if t2 >= 0.5 * target_s or n >= len(kept):
            break
        n = int(min(len(kept), n * min(8.0, max(2.0, target_s / max(t2, 1e-3)))))
    fl = per_row * float(visible_keys(batch, rows).sum())
    cores = _blas_threads()
    base = {"value": round(fl / t2 / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{n} of the {batch.T} query rows of {batch.name} (seeded random choice), all "
                      f"{batch.Hq} heads, {fl / 1e9:.1f} GFLOP in {t2:.1f} s, numpy float64 with BLAS "
                      f"threads={cores}; {np.__version__}"}
    pos = np.searchsorted(kept, rows)
    return base, _parity(rows, ro, rl, gpu_out[pos], gpu_lse[pos], 2e-2, batch)


PHASE_NAMES = ((0, "start"), (7, "lens and table staged"), (1, "block prefix"), (10, "table window"),
               (2, "new rows stored"), (3, "split pieces streamed"), (5, "partial stores complete"),
               (6, "merge counters"), (4, "published and merged"), (15, "end"))


def decode_phases(args) -> None:
    """Per-phase timestamps of the fused decode step at the decode workload:
    the library built with the decode kernel's phase probes (libkvstore_phases.so)
    runs GRAPH back-to-back steps from a HIP graph, rotating the replicas; after
    each replay the probes of its last launch are read (100 MHz device clock,
    microseconds from the first workgroup's start).  Prints one JSON line."""
    import ctypes

    import numpy as np
    import torch

    import attention_kv_store_amd._lib as L

    lib = L.load(L.PHASES_LIB_PATH)
    lib.kvs_phase_times.argtypes = [ctypes.c_void_p]
    lib.kvs_phase_times.restype = ctypes.c_int
    lib.kvs_phase_clear.argtypes = []
    lib.kvs_phase_clear.restype = ctypes.c_int
    import attention_kv_store_amd as kvs
    from workloads import paged_decode_bf16

    dec = paged_decode_bf16()
    w = Workload(dec, args.replicas)
    for i in range(8):
        w.append_attend(i)
    torch.cuda.synchronize()
    graph_len = 6
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(graph_len):
            w.append_attend(i)
    buf = np.zeros((4096, 16), dtype=np.uint64)
    reps = []
    for _ in range(5):
        if lib.kvs_phase_clear() != 0:
            raise SystemExit("kvs_phase_clear failed")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        if lib.kvs_phase_times(buf.ctypes.data_as(ctypes.c_void_p)) != 0:
            raise SystemExit("kvs_phase_times failed")
        nwg = int(kvs.last_dispatch().split("grid=(")[1].split(",")[0])
        t = buf[:nwg].astype(np.int64)
        rel = (t - t[:, 0].min()) / 100.0
        rel[t == 0] = np.nan
        ph = {}
        for k, name in PHASE_NAMES:
            col = rel[:, k][~np.isnan(rel[:, k])]
            if col.size:
                ph[name] = {"n": int(col.size), "min": round(float(col.min()), 2), "p50": round(float(np.median(col)), 2),
                            "p90": round(float(np.percentile(col, 90)), 2), "max": round(float(col.max()), 2)}
        end = rel[:, 15]
        late = np.argsort(np.nan_to_num(end))[-16:]
        merging = int(np.sum((buf[:nwg, 8] & 3) > 0))
        reps.append({"launch_us": round(e0.elapsed_time(e1) * 1e3 / graph_len, 2), "workgroups": nwg,
                     "merging_workgroups": merging, "phases_us": ph,
                     "latest_16_workgroups_xcd": sorted(int(x) % 8 for x in late)})
        log(f"decode phases: {reps[-1]['launch_us']} us per launch, end p50 {ph['end']['p50']} max {ph['end']['max']}")
    print(json.dumps({"decode_phases": {"workload": "paged_decode_bf16", "step": "attn_decode_append_paged",
                                        "dispatch": kvs.last_dispatch(), "graph_launches": graph_len,
                                        "replays": reps}}))


# the prefill configurations measured: workload, device replicas rotated so
# that the working set exceeds the 256 MB Infinity Cache, most timed steps
PREFILL_CONFIGS = (
    ("causal_prefill_bf16", 4, 500),
    ("extend_prefill_bf16", 2, 500),
    ("long_prefill_bf16", 1, 50),
)
PARITY_ROWS = 4096   # GPU output rows kept for the parity check (a seeded random order)


def prefill_line(name, replicas, cap, args):
    """One prefill configuration: each step stores the batch's new K/V rows
    (kv_store_paged) and runs attn_varlen_paged; the attention launch alone
    gives roofline.achieved.  Returns the line's entry and the GPU's timed
    outputs on PARITY_ROWS seeded rows (for the CPU leg's parity check)."""
    import numpy as np
    import torch

    import attention_kv_store_amd as kvs
    from workloads import NAMED, attention_flops, io_bytes

    b = NAMED[name]()
    w = Workload(b, replicas)
    steps = min(cap, max(1, args.steps // 4))
    warm = max(1, min(cap, args.warmup // 4))
    pms, pattn, _, pstats = time_steps(w, steps, warm, eager=args.eager)
    disp = kvs.last_dispatch()
    fl = attention_flops(b)
    tf = fl / (pattn * 1e-3) / 1e12
    log(f"{name}: {pms*1e3:.2f} us/step, attention {pattn*1e3:.2f} us -> {tf:.1f} TFLOP/s ({disp})")
    entry = {
        "workload": name, "query_rows": b.T, "sequences": b.B, "metric": "attention TFLOP/s",
        "unit": "TFLOP/s", "ms_per_step": round(pms, 6), "steps": steps, "replicas": replicas,
        "dispatch": disp, "replay_stats": pstats,
        "roofline": {
            "bound": "mfma", "kernel": COUNTED[name][0], "achieved": round(tf, 3), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tf / BF16_PEAK_TFLOPS, 4), "traffic": _traffic(COUNTED[name][1], name),
            "flops_per_launch": fl, "avg_launch_us": round(pattn * 1e3, 3), "io_bytes_per_launch": io_bytes(b),
        },
    }
    perm = np.random.default_rng(1234).permutation(b.T)
    keep = np.sort(perm[:PARITY_ROWS])
    idx = torch.from_numpy(keep).cuda()
    _, _, _, _, out, lse = w.reps[0]
    gout = out.index_select(0, idx).float().cpu().numpy().astype(np.float64)
    glse = lse.index_select(0, idx).float().cpu().numpy().astype(np.float64)
    del w
    torch.cuda.empty_cache()
    return entry, (b, perm, keep, gout, glse)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--eager", action="store_true", help="time plain launches instead of graph replays")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the headline decode and prefill workloads (no warm, graph-runner, mixed or peak "
                         "figures): the profiler runs use it so each kernel name covers one workload")
    ap.add_argument("--summarize-counters", nargs="+", metavar="WORKLOAD=READ_CSV,WRITE_CSV",
                    help="write profiles/traffic_counters.json from rocprofv3 --pmc runs and exit")
    ap.add_argument("--prefill", default=",".join(n for n, _, _ in PREFILL_CONFIGS),
                    help="comma-separated prefill configurations to run (the profiler runs take one at a "
                         "time where two share a kernel)")
    ap.add_argument("--counter-command", default="", help="command line recorded with --summarize-counters")
    ap.add_argument("--decode-phases", action="store_true",
                    help="print the decode kernel's per-phase timestamps (libkvstore_phases.so) and exit")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.counter_command)
        return
    if args.decode_phases:
        decode_phases(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the attention would shard by KV head, with no exchange between GPUs).", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import attention_kv_store_amd as kvs
    from workloads import attention_flops, io_bytes, kv_bytes, paged_decode_bf16

    dec = paged_decode_bf16()
    prefill_outputs = {}
    log(f"decode batch: B={dec.B} sum(Lk)={int(dec.k_lens.sum())} K+V={kv_bytes(dec)/1e6:.1f} MB")
    w = Workload(dec, args.replicas)
    kvb = kv_bytes(dec)
    # the first call of the process (module load and first dispatch), by itself
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    w.append_attend(0)
    c1.record()
    torch.cuda.synchronize()
    cold_ms = c0.elapsed_time(c1)
    sms, sattn_ms, _, sstats = time_steps(w, args.steps, args.warmup, eager=args.eager)
    sdispatch = kvs.last_dispatch()
    log(f"decode, two calls: {sms*1e3:.2f} us/step, attention {sattn_ms*1e3:.2f} us ({sdispatch})")
    ms, attn_ms, wall, stats = time_steps(w, args.steps, args.warmup, fused=True, eager=args.eager)
    dispatch = kvs.last_dispatch()
    value = kvb / (ms * 1e-3) / 1e9
    achieved = kvb / (attn_ms * 1e-3) / 1e9
    log(f"decode, fused: {ms*1e3:.2f} us/step, launch {attn_ms*1e3:.2f} us -> {achieved:.0f} GB/s ({dispatch})")
    traffic = _traffic(COUNTED["paged_decode_bf16"][1], "paged_decode_bf16")
    # the outputs of the last timed step (every replica computes the same)
    dec_out = w.reps[0][4].float().cpu().numpy().astype("float64")
    dec_lse = w.reps[0][5].cpu().numpy().astype("float64")
    line = {
        "metric": "prefill attn TFLOP/s (% bf16 MFMA peak); decode KV GB/s (% HBM peak)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) q/k/v, seeded lengths and shuffled block table)",
        "config": {
            "workload": "paged_decode_bf16",
            "batch_sequences": dec.B, "query_rows": dec.T, "context_min": int(dec.k_lens.min()),
            "context_max": int(dec.k_lens.max()), "context_sum": int(dec.k_lens.sum()),
            "q_heads": dec.Hq, "kv_heads": dec.Hkv, "head_dim": dec.D, "page_size": 16,
            "replicas": args.replicas,
            "step": "attn_decode_append_paged (new K/V rows stored and attended in one launch)",
            "timing": "eager launches" if args.eager else f"HIP graph replays ({_graph_len(args.steps)} steps per graph)",
            "dispatch": dispatch,
        },
        "two_calls": {
            "step": "kv_store_paged(new rows) + attn_varlen_paged",
            "ms_per_step": round(sms, 6), "value": round(kvb / (sms * 1e-3) / 1e9, 2), "unit": "GB/s",
            "attention_us": round(sattn_ms * 1e3, 3), "dispatch": sdispatch, "replay_stats": sstats,
        },
        "replay_stats": stats,
        "cold_first_call_ms": round(cold_ms, 3),
        "roofline": {
            "bound": "hbm",
            "kernel": COUNTED["paged_decode_bf16"][0] + " (the one launch of each attn_decode_append_paged call)",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": kvb,
            "avg_launch_us": round(attn_ms * 1e3, 3),
            "io_bytes_per_launch": io_bytes(dec),
        },
    }
    del w
    torch.cuda.empty_cache()
    if not args.no_extras:
        # the same decode steps on one replica: K/V may then stay in the 256 MB
        # Infinity Cache between steps (labelled warm; the headline rotates replicas)
        w1 = Workload(dec, 1)
        wms, _, _, _ = time_steps(w1, max(100, args.steps // 4), max(1, args.warmup // 4), fused=True,
                                  eager=args.eager)
        line["warm_one_replica"] = {"ms_per_step": round(wms, 6), "value": round(kvb / (wms * 1e-3) / 1e9, 2),
                                    "unit": "GB/s", "note": "1 replica: K/V can stay in the Infinity Cache"}
        del w1
        torch.cuda.empty_cache()

        # graph runner (decode steps replayed from per-bucket graphs): the first 50
        # sequences of the batch padded to the 64-row bucket with dummy rows, and
        # all 64 -- replays only (inputs already in the bucket's buffers)
        line["graph_runner"] = runner_replays(dec, args)
        log(f"graph runner: {line['graph_runner']}")

    if not args.no_prefill:
        # causal prefill (16 x 512), extend over a cached prefix (8 sequences),
        # one 32768-token prompt
        line["prefill"] = {}
        chosen = [x for x in args.prefill.split(",") if x]
        unknown = set(chosen) - {n for n, _, _ in PREFILL_CONFIGS}
        if unknown:
            raise SystemExit(f"unknown prefill configurations {sorted(unknown)}")
        for name, reps, cap in PREFILL_CONFIGS:
            if name not in chosen:
                continue
            entry, keep = prefill_line(name, reps, cap, args)
            line["prefill"][name] = entry
            prefill_outputs[name] = keep

    if not args.no_prefill and not args.no_extras:
        # a mixed serving step in one launch: 2 prompts x 256 new tokens and 30
        # decode rows over 128..2048-token contexts (M = 542 rows); it runs on
        # the prefill/extend kernel (T != B)
        from workloads import mixed_prefill_decode_bf16
        mix = mixed_prefill_decode_bf16()
        wm = Workload(mix, args.replicas)
        msteps = max(1, args.steps // 4)
        mms, mattn, _, mstats = time_steps(wm, msteps, max(1, args.warmup // 4), eager=args.eager)
        line["mixed"] = {
            "workload": "mixed_prefill_decode_bf16", "query_rows": mix.T, "sequences": mix.B,
            "avg_launch_us": round(mattn * 1e3, 3),
            "TFLOPs": round(attention_flops(mix) / (mattn * 1e-3) / 1e12, 3),
            "kv_GBs": round(kv_bytes(mix) / (mattn * 1e-3) / 1e9, 2),
            "flops_per_launch": attention_flops(mix), "kv_bytes_per_launch": kv_bytes(mix),
            "dispatch": kvs.last_dispatch(), "replay_stats": mstats,
        }
        del wm
        torch.cuda.empty_cache()
        # the same batch with its 30 decode rows declared (decode_tail): prefill
        # kernel on the 2 prompts, decode kernel on the 30 decode rows
        n_dec = int((mix.q_lens == 1).sum())
        wm = Workload(mix, args.replicas, decode_tail=n_dec)
        tms, tattn, _, tstats = time_steps(wm, msteps, max(1, args.warmup // 4), eager=args.eager)
        line["mixed"]["with_decode_tail"] = {
            "decode_tail": n_dec, "us_per_call": round(tattn * 1e3, 3),
            "kv_GBs": round(kv_bytes(mix) / (tattn * 1e-3) / 1e9, 2),
            "dispatch": kvs.last_dispatch(), "replay_stats": tstats,
        }
        log(f"mixed: {line['mixed']}")
        del wm
        torch.cuda.empty_cache()

    if not args.no_prefill and not args.no_extras:
        # sliding-window variants: the decode workload under a 512-key window
        # (fused step) and 4 x 4096-token prompts under a 1024-key window
        from workloads import sliding_window_decode_bf16, sliding_window_prefill_bf16
        sw = {}
        wd = sliding_window_decode_bf16()
        ww = Workload(wd, args.replicas)
        dms, _, _, dstats = time_steps(ww, args.steps, args.warmup, fused=True, eager=args.eager)
        sw["decode"] = {
            "workload": "sliding_window_decode_bf16", "window": wd.window, "step": "attn_decode_append_paged_window",
            "avg_launch_us": round(dms * 1e3, 3), "kv_bytes_per_launch": kv_bytes(wd),
            "GBs": round(kv_bytes(wd) / (dms * 1e-3) / 1e9, 2),
            "frac": round(kv_bytes(wd) / (dms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "dispatch": kvs.last_dispatch(), "replay_stats": dstats,
        }
        del ww
        torch.cuda.empty_cache()
        wpf = sliding_window_prefill_bf16()
        ww = Workload(wpf, args.replicas)
        psteps = max(1, args.steps // 4)
        _, wattn, _, wstats = time_steps(ww, psteps, max(1, args.warmup // 4), eager=args.eager)
        sw["prefill"] = {
            "workload": "sliding_window_prefill_bf16", "window": wpf.window, "query_rows": wpf.T,
            "avg_launch_us": round(wattn * 1e3, 3), "flops_per_launch": attention_flops(wpf),
            "TFLOPs": round(attention_flops(wpf) / (wattn * 1e-3) / 1e12, 3),
            "frac": round(attention_flops(wpf) / (wattn * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "dispatch": kvs.last_dispatch(), "replay_stats": wstats,
        }
        del ww
        torch.cuda.empty_cache()
        line["sliding_window"] = sw
        log(f"sliding window: {sw}")

    if not args.no_extras:
        from workloads import causal_prefill_bf16 as _cp
        line["fp8_kv"] = {"decode": fp8_line(dec, args), "prefill": fp8_line(_cp(), args, n=40)}
        line["fp8_kv"]["decode_step"] = fp8_step_line(dec, args)
        log(f"fp8 cache: {line['fp8_kv']}")
        line["int8_kv"] = {"decode": fp8_line(dec, args, fmt="int8"), "prefill": fp8_line(_cp(), args, n=40, fmt="int8"),
                           "decode_step": fp8_step_line(dec, args, fmt="int8")}
        log(f"int8 cache: {line['int8_kv']}")
        line["decode_context_sweep"] = context_sweep(args)
        log(f"decode context sweep: {line['decode_context_sweep']}")
        line["rope_store"] = rope_store_line(args)
        line["rope_decode_step"] = rope_decode_line(dec, args)
        log(f"rope decode step: {line['rope_decode_step']}")
        log(f"rope + store: {line['rope_store']}")

    if not args.no_extras:
        peaks = measure_peaks()
        line["measured_peaks"] = peaks
        line["roofline"]["frac_of_measured_copy"] = round(achieved / peaks["copy_GBs"], 4)
        for entry in line.get("prefill", {}).values():
            entry["roofline"]["frac_of_measured_mfma"] = round(entry["roofline"]["achieved"] / peaks["bf16_mfma_TFLOPs"], 4)
        log(f"measured peaks: {peaks}")
    line["env"] = environment()

    if not args.no_cpu_baseline:
        # the oracle on the host cores (rank 0, one GPU), on the same inputs;
        # the rows it computes also check the GPU's timed outputs
        log("timing the CPU oracle ...")
        line["cpu_baseline"], line["parity"] = cpu_baseline(dec, dec_out, dec_lse)
        log(f"decode: cpu {line['cpu_baseline']['value']} GB/s, parity {line['parity']}")
        for name, (b, perm, kept, gout, glse) in prefill_outputs.items():
            base, par = cpu_baseline_prefill(b, perm, kept, gout, glse)
            line["prefill"][name]["cpu_baseline"] = base
            line["prefill"][name]["parity"] = par
            log(f"{name}: cpu {base['value']} TFLOP/s ({base['sample']}), parity {par}")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
