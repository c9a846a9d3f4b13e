#!/usr/bin/env python3
"""Benchmark of the paged varlen attention path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass of the whole path over one batch: kv_store_paged of the
batch's new K/V rows, then attn_varlen_paged.  The headline workload is the
paged decode batch (64 sequences x 1 query row, contexts uniform in
[128, 2048], 32 query / 8 KV heads, head dim 64, bf16, 16-token pages,
shuffled blocks); its metric is K+V bytes read per second.  The causal prefill
batch (16 x 512 tokens, 32/8 heads, head dim 128, bf16) is measured the same
way and reported under "prefill" in attention TFLOP/s.

Timing follows the device-event method of Transformer 추론 커널 (3/10), §26:
warm-up launches, then K back-to-back steps between two events on the stream.
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


def _src_sha(name: str) -> str:
    path = os.path.join(ROOT, "attention_kv_store_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def _traffic(kernel_src: str, workload: str):
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

    def __init__(self, batch, replicas: int):
        import torch
        from tests.gpu_side import to_device

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
        need = kvs.workspace_size(db.q, db.k_cache, db.block_table)
        self.ws = [torch.zeros(max(need, 1), dtype=torch.uint8, device="cuda") for _ in range(replicas)]
        torch.cuda.synchronize()

    def store(self, i):
        db, kn, vn, sl, _, _ = self.reps[i % len(self.reps)]
        self.kvs.kv_store_paged(kn, vn, sl, db.k_cache, db.v_cache)

    def attend(self, i):
        r = i % len(self.reps)
        db, _, _, _, out, lse = self.reps[r]
        self.kvs.attn_varlen_paged(db.q, db.k_cache, db.v_cache, db.block_table, db.cu_seqlens_q,
                                   db.seqlens_k, db.scale, db.causal, out=out, lse=lse, workspace=self.ws[r])


def time_steps(w: Workload, steps: int, warmup: int):
    """K timed steps between two events; per-phase events inside the region
    give the attention call's own average duration on the same stream."""
    import torch

    for i in range(warmup):
        w.store(i)
        w.attend(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        w.store(i)
        ev[i][0].record()
        w.attend(i)
        ev[i][1].record()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / steps
    attn = [a.elapsed_time(b) for a, b in ev]
    attn_ms = sum(attn) / steps
    return ms_step, attn_ms, wall


def cpu_baseline(batch, target_s: float = 10.0):
    """The oracle, untuned, on the same batch: repeated whole-batch calls until
    about target_s seconds of host time; K+V bytes / second."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import attention_oracle
    from tests.oracle_side import oracle_pool
    from workloads import kv_bytes

    kc, vc = oracle_pool(batch)
    n, t = 0, 0.0
    while t < target_s:
        t0 = time.perf_counter()
        attention_oracle(batch.q, kc, vc, batch.block_table, batch.cu_seqlens_q, batch.k_lens,
                         batch.scale, batch.causal)
        t += time.perf_counter() - t0
        n += 1
    info = threadpool_info()
    cores = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] or [1])
    return {"value": round(kv_bytes(batch) * n / t / 1e9, 4), "unit": "GB/s", "cores": int(cores),
            "kind": "oracle",
            "sample": f"whole paged_decode_bf16 batch (64 rows, all heads), {n} calls in {t:.1f} s, "
                      f"numpy float64 with BLAS threads={cores}; {np.__version__}"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the attention shards by KV head with no exchange; see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import attention_kv_store_amd as kvs
    from workloads import attention_flops, causal_prefill_bf16, io_bytes, kv_bytes, paged_decode_bf16

    dec = paged_decode_bf16()
    log(f"decode batch: B={dec.B} sum(Lk)={int(dec.k_lens.sum())} K+V={kv_bytes(dec)/1e6:.1f} MB")
    w = Workload(dec, args.replicas)
    ms, attn_ms, wall = time_steps(w, args.steps, args.warmup)
    dispatch = kvs.last_dispatch()
    kvb = kv_bytes(dec)
    value = kvb / (ms * 1e-3) / 1e9
    achieved = kvb / (attn_ms * 1e-3) / 1e9
    log(f"decode: {ms*1e3:.2f} us/step, attention {attn_ms*1e3:.2f} us -> {achieved:.0f} GB/s ({dispatch})")
    traffic = _traffic("decode.hip", "paged_decode_bf16")
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
            "replicas": args.replicas, "step": "kv_store_paged(new rows) + attn_varlen_paged",
            "dispatch": dispatch,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": "decode_split_kernel + decode_merge_kernel (one attn_varlen_paged call)",
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

    if not args.no_prefill:
        pre = causal_prefill_bf16()
        wp = Workload(pre, args.replicas)
        psteps = max(1, args.steps // 4)
        pms, pattn, _ = time_steps(wp, psteps, max(1, args.warmup // 4))
        pdisp = kvs.last_dispatch()
        fl = attention_flops(pre)
        tf = fl / (pattn * 1e-3) / 1e12
        log(f"prefill: {pms*1e3:.2f} us/step, attention {pattn*1e3:.2f} us -> {tf:.1f} TFLOP/s ({pdisp})")
        line["prefill"] = {
            "workload": "causal_prefill_bf16",
            "metric": "attention TFLOP/s", "unit": "TFLOP/s", "bound": "mfma",
            "achieved": round(tf, 3), "peak": BF16_PEAK_TFLOPS, "frac": round(tf / BF16_PEAK_TFLOPS, 4),
            "flops_per_launch": fl, "avg_launch_us": round(pattn * 1e3, 3),
            "ms_per_step": round(pms, 6), "steps": psteps,
            "traffic": _traffic("prefill.hip", "causal_prefill_bf16"),
            "dispatch": pdisp,
        }
        del wp
        torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        line["cpu_baseline"] = cpu_baseline(dec)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
