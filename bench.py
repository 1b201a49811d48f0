#!/usr/bin/env python3
"""Benchmark of paged BSR attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one pass of the hot path over one batch of the batch paged decode
workload (64 requests, GQA 32/8, head_dim 128, page 16, bf16, kv_len uniform on
[512, 4096]): the CPU plan of the batch, its upload, the persistent decode
kernel and the merge of split tiles. Inputs are resident in HBM before the timed
region; the K/V pools are replicated and rotated so that no step can hit data
a previous step left in the 256 MB last-level cache.

Prints one JSON line. ``value`` is achieved HBM throughput of the step in TB/s
(algorithmic bytes: valid K/V tokens + q + o + lse + page indices).
``roofline`` is the decode kernel(s) alone, timed with HIP events on their
stream. ``append`` is the ragged causal append workload (16 requests, qo
U{128..1024} onto kv U{1024..8192}, GQA 32/8, bf16) in TFLOP/s of causal
algorithmic work. ``cpu_baseline`` is the fp64 oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_TBS = 8.0           # MI355X HBM3E, TB/s
MFMA_BF16_PEAK_TFLOPS = 2516.6  # dense bf16 MFMA, 256 CU x 4096 flop/clk x 2.4 GHz


def decode_bytes(w, batch_ids=None) -> int:
    """Algorithmic bytes of a decode batch: each valid K/V token once, q, o, lse, indices."""
    kv = w.kv
    ids = range(w.batch) if batch_ids is None else batch_ids
    tokens = int(sum(int(kv.kv_len[b]) for b in ids))
    pages = int(sum(int(kv.kv_indptr[b + 1] - kv.kv_indptr[b]) for b in ids))
    n = len(list(ids))
    elt = 2
    kvb = tokens * w.num_kv_heads * w.head_dim * 2 * elt
    qo = 2 * n * w.num_qo_heads * w.head_dim * elt
    return kvb + qo + n * w.num_qo_heads * 4 + pages * 4 + (n + 1) * 4 + n * 4


def append_flops(w) -> float:
    """Causal algorithmic FLOP: 4 * d * Hq per visible (query, key) pair."""
    qo = np.diff(w.qo_indptr).astype(np.float64)
    kv = w.kv.kv_len.astype(np.float64)
    pairs = (qo * (kv - qo) + qo * (qo + 1) / 2).sum() if w.causal else (qo * kv).sum()
    return 4.0 * w.head_dim * w.num_qo_heads * pairs


def cpu_baseline_decode(w, budget_s: float = 12.0):
    """The fp64 oracle on whole requests until ~budget_s of CPU work (1 BLAS thread)."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as ora
    done, t_used = [], 0.0
    with threadpool_limits(limits=1):
        for b in range(w.batch):
            t0 = time.perf_counter()
            ora.decode_workload(w, batch_ids=[b])
            t_used += time.perf_counter() - t0
            done.append(b)
            if t_used >= budget_s:
                break
    by = decode_bytes(w, done)
    return {"value": by / t_used / 1e12, "unit": "TB/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(done)} of {w.batch} requests of the same batch "
                      f"({by / 1e6:.1f} MB algorithmic) in {t_used:.1f} s, fp64 NumPy, 1 thread"}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workers", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-append", action="store_true")
    ap.add_argument("--part", choices=["all", "decode", "append"], default="all",
                    help="decode or append alone (profiling); 'all' is the benchmark line")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the paged attention path has no multi-GPU "
              "component (each GPU would run its own share with no exchange); use --gpus 1",
              file=sys.stderr)
        return 2

    import torch

    import attention_bsr_paged_amd as abp
    from attention_bsr_paged_amd import workloads as wl

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    abp.load_library()
    if args.part == "append":
        print(json.dumps(bench_append(abp, wl, torch, dev, args.steps, args.warmup)), flush=True)
        return 0

    # ------------------------------------------------------------------ decode
    w = wl.batch_decode_gqa()
    kv = w.kv
    by = decode_bytes(w)
    pool_bytes = kv.k_pages.nbytes + kv.v_pages.nbytes
    copies = max(2, math.ceil(2 * 2 ** 30 / pool_bytes))
    k0 = wl.to_torch(kv.k_pages, w.dtype, dev)
    v0 = wl.to_torch(kv.v_pages, w.dtype, dev)
    ks = [k0] + [k0.clone() for _ in range(copies - 1)]
    vs = [v0] + [v0.clone() for _ in range(copies - 1)]
    q = wl.to_torch(w.q, w.dtype, dev)
    indptr = torch.from_numpy(kv.kv_indptr).to(dev)
    indices = torch.from_numpy(kv.kv_indices).to(dev)
    lpl = torch.from_numpy(kv.kv_last_page_len).to(dev)
    params = abp.make_params(w.num_qo_heads, w.num_kv_heads, w.head_dim, kv.page_size,
                             torch.bfloat16)
    dec = abp.BatchDecode(params, max_batch=w.batch, num_workers=args.workers, device=dev)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    K, Wm = args.steps, args.warmup
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]

    def step(i, evs=None):
        dec.plan(kv.kv_indptr, kv.kv_last_page_len, stream=stream)
        if evs:
            evs[0].record(stream)
        dec.run(q, ks[i % copies], vs[i % copies], indptr, indices, lpl, o=o, lse=lse,
                stream=stream)
        if evs:
            evs[1].record(stream)

    for i in range(Wm):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(i, ev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    kern_ms = np.array([a.elapsed_time(b) for a, b in ev])
    kern_avg = float(kern_ms.mean())
    plan = dec.plan_struct

    t_plan0 = time.perf_counter()
    for _ in range(50):
        dec.plan(kv.kv_indptr, kv.kv_last_page_len, stream=stream)
    plan_us = (time.perf_counter() - t_plan0) / 50 * 1e6
    torch.cuda.synchronize()

    value = by / (ms_step * 1e-3) / 1e12
    achieved = by / (kern_avg * 1e-3) / 1e9
    out = {
        "metric": "paged-decode achieved HBM TB/s (% of peak) + causal-append TFLOPS, bf16 GQA",
        "value": round(value, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "batch": w.batch,
            "num_qo_heads": w.num_qo_heads,
            "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim,
            "page_size": kv.page_size,
            "kv_tokens": int(kv.kv_len.sum()),
            "algorithmic_bytes": by,
            "workers": plan.num_workers,
            "segments": plan.num_segments,
            "merged_tiles": plan.num_merges,
            "kv_pool_copies": copies,
            "parallelism": "single GPU",
        },
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_TBS, 2),
        "plan_us": round(plan_us, 2),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_TBS * 1e3,
            "unit": "GB/s",
            "frac": round(achieved / (HBM_PEAK_TBS * 1e3), 4),
            "traffic": None,
            "kernel": "decode_kernel + plan_merge_kernel (one run() call)",
            "avg_launch_us": round(kern_avg * 1e3, 2),
            "p10_us": round(float(np.percentile(kern_ms, 10)) * 1e3, 2),
            "p90_us": round(float(np.percentile(kern_ms, 90)) * 1e3, 2),
        },
    }

    # ------------------------------------------------------------------ append
    if not args.no_append and args.part == "all":
        try:
            out["append"] = bench_append(abp, wl, torch, dev, max(20, K // 4), 5)
        except abp.AbpError as e:
            out["append"] = {"error": str(e)}

    # ------------------------------------------------------------- CPU baseline
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(w)
    print(json.dumps(out), flush=True)
    return 0


def bench_append(abp, wl, torch, dev, K, Wm):
    w = wl.ragged_append_causal()
    kv = w.kv
    flops = append_flops(w)
    q = wl.to_torch(w.q, w.dtype, dev)
    k = wl.to_torch(kv.k_pages, w.dtype, dev)
    v = wl.to_torch(kv.v_pages, w.dtype, dev)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    qo, indptr, indices, lpl = i32(w.qo_indptr), i32(kv.kv_indptr), i32(kv.kv_indices), \
        i32(kv.kv_last_page_len)
    params = abp.make_params(w.num_qo_heads, w.num_kv_heads, w.head_dim, kv.page_size,
                             torch.bfloat16, causal=True)
    app = abp.BatchAppend(params, max_batch=w.batch, max_qo_tokens=int(w.qo_indptr[-1]),
                          device=dev)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream(dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(K)]
    for i in range(Wm + K):
        app.plan(w.qo_indptr, kv.kv_indptr, kv.kv_last_page_len, stream=s)
        e = evs[i - Wm] if i >= Wm else None
        if e:
            e[0].record(s)
        app.run(q, k, v, qo, indptr, indices, lpl, o=o, lse=lse, stream=s)
        if e:
            e[1].record(s)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in evs])
    avg = float(ms.mean())
    tf = flops / (avg * 1e-3) / 1e12
    return {
        "workload": w.name,
        "value": round(tf, 2),
        "unit": "TFLOP/s",
        "causal_flop": flops,
        "avg_run_us": round(avg * 1e3, 2),
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None},
        "workers": app.plan_struct.num_workers,
    }


if __name__ == "__main__":
    sys.exit(main())
