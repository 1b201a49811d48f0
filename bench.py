#!/usr/bin/env python3
"""Benchmark of paged BSR attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--part all|decode|append|single|skewed|cascade|copy|bsr|page_append|fp8_decode]

A step is one pass of the hot path over one batch of the batch paged decode
workload (64 requests, GQA 32/8, head_dim 128, page 16, bf16, kv_len uniform on
[512, 4096]): the CPU plan of the batch (validation, kv lengths, Stream-K
partition), its upload, the persistent decode kernel and the merge of split
tiles. Inputs are resident in HBM before the timed region; the K/V pools are
replicated and rotated (at least 2 GiB in all) so that no step reads data a
previous step left in the 256 MB last-level cache. After the K timed steps,
each leg runs max(100, K) more runs bracketed one by one by HIP events on their
stream (median, p10 and p90 of the run), sampling the engine clock meanwhile.

Prints one JSON line. ``value`` is achieved HBM throughput of the whole step in
TB/s (algorithmic bytes: each valid K/V token once, plus q, o, lse and the
page indices). ``roofline`` is the decode run alone (decode kernel + merge
kernel), timed with HIP events on the stream it is launched on. ``append`` is
the ragged causal append workload (16 requests, qo U{128..1024} onto kv
U{1024..8192}, GQA 32/8, bf16) in TFLOP/s of visible (unmasked) work;
``configs`` holds the single-request, skewed-batch and cascade+RoPE decode
workloads; ``next`` holds block-sparse attention (8192 x 8192, row blocks of
64, column blocks of 16, a quarter of the blocks, TFLOP/s of unmasked work)
the page append of 16 requests' new tokens (TB/s of rows read + written) and
the batch decode shape over an fp8 (e4m3) KV cache (TB/s of its one-byte K/V).
``cpu_baseline`` is the fp64 oracle on a bounded sample of the batch decode
workload, on the host cores of the same machine (and of each other leg).

``--part copy`` times a plain 1 GiB device copy (read + write of known size);
its counter readings calibrate FETCH_SIZE / WRITE_SIZE for the traffic figure.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_TBS = 8.0              # MI355X HBM3E, TB/s
MFMA_BF16_PEAK_TFLOPS = 2516.6  # dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
FLUSH_BYTES = 2 * 2 ** 30       # K/V replicas rotated per step (>> 256 MB MALL)

# Counter readings (FETCH_SIZE / WRITE_SIZE) of the decode run and of a plain
# copy, recorded by rocprofv3; valid only while the kernel sources hash the same.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_run_batch_decode_traffic.txt")
DECODE_SOURCES = ["decode.hip", "decode_mfma.hip", "decode_mfma_impl.h", "merge.hip", "common.h", "kernels.h", "layout.h"]


PAGE_APPEND_TRAFFIC_FILE = os.path.join(ROOT, "profiles",
                                        "page_append_kernel_ragged_page_append_traffic.txt")
PAGE_APPEND_SOURCES = ["page_append.hip"]


def source_hash(names=DECODE_SOURCES) -> str:
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "attention_bsr_paged_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(path=TRAFFIC_FILE, sources=DECODE_SOURCES):
    """Bytes per run from a committed counter summary, or None when the summary
    is absent or the kernel sources changed since it was taken."""
    try:
        text = open(path).read()
    except OSError:
        return None
    m = re.search(r"^TRAFFIC (\{.*\})\s*$", text, re.M)
    if not m:
        return None
    rec = json.loads(m.group(1))
    if rec.get("source_sha256_16") != source_hash(sources):
        return None
    return rec


# ----------------------------------------------------------------------------
# algorithmic work
# ----------------------------------------------------------------------------
def decode_bytes(w, batch_ids=None) -> int:
    """Algorithmic bytes of a decode batch: each valid K/V token once, q, o, lse, indices."""
    kv = w.kv
    ids = list(range(w.batch) if batch_ids is None else batch_ids)
    tokens = int(sum(int(kv.kv_len[b]) for b in ids))
    pages = int(sum(int(kv.kv_indptr[b + 1] - kv.kv_indptr[b]) for b in ids))
    n = len(ids)
    elt = 2
    kv_elt = 1 if kv.dtype == "fp8_e4m3" else 2   # e4m3 pages: one byte per element
    kvb = tokens * w.num_kv_heads * w.head_dim * 2 * kv_elt
    qo = 2 * n * w.num_qo_heads * w.head_dim * elt
    return kvb + qo + n * w.num_qo_heads * 4 + pages * 4 + (n + 1) * 4 + n * 4


def cascade_bytes(w) -> int:
    """The shared prefix once, every suffix token once, q, o, lse and indices."""
    pre = w.prefix
    pre_tokens = int(pre.kv_len.sum())
    kv_row = w.num_kv_heads * w.head_dim * 2 * 2
    return decode_bytes(w) + pre_tokens * kv_row + int(pre.kv_indptr[-1]) * 4


def append_flops(w, token_ids=None) -> float:
    """Causal algorithmic FLOP: 4 * d * Hq per visible (query, key) pair."""
    qo = np.diff(w.qo_indptr).astype(np.int64)
    kv = w.kv.kv_len.astype(np.int64)
    if token_ids is None:
        if w.causal:
            pairs = (qo * (kv - qo) + qo * (qo + 1) // 2).sum()
        else:
            pairs = (qo * kv).sum()
    else:
        pairs = 0
        for t in token_ids:
            b = int(np.searchsorted(w.qo_indptr, t, side="right") - 1)
            i = t - int(w.qo_indptr[b])
            pairs += int(kv[b] - qo[b] + i + 1) if w.causal else int(kv[b])
    return 4.0 * w.head_dim * w.num_qo_heads * float(pairs)


# ----------------------------------------------------------------------------
# timing helpers
# ----------------------------------------------------------------------------
def _stats_ms(ms: np.ndarray) -> dict:
    return {"avg_us": round(float(ms.mean()) * 1e3, 2),
            "median_us": round(float(np.median(ms)) * 1e3, 2),
            "p10_us": round(float(np.percentile(ms, 10)) * 1e3, 2),
            "p90_us": round(float(np.percentile(ms, 90)) * 1e3, 2)}


SAMPLES = 100     # runs bracketed by HIP events per leg, after the timed steps


def _sclk_path():
    """sysfs file listing the GPU's engine clock levels, the current one marked
    with '*' (one GPU per box here; None when it cannot be read)."""
    import glob
    paths = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
    vis = os.environ.get("HIP_VISIBLE_DEVICES") or os.environ.get("ROCR_VISIBLE_DEVICES")
    if len(paths) == 1 or (paths and not vis):
        return paths[0] if len(paths) == 1 else None
    return None


class ClockSampler:
    """Samples the current engine clock (MHz) from sysfs every `period` seconds
    on a background thread while a leg's runs execute."""

    def __init__(self, period: float = 0.002):
        self.path = _sclk_path()
        self.period = period
        self.samples = []
        self._stop = None
        self._thread = None

    def _read(self):
        try:
            with open(self.path) as f:
                for line in f:
                    if "*" in line:
                        m = re.search(r"(\d+)\s*[Mm][Hh]z", line)
                        return int(m.group(1)) if m else None
        except OSError:
            return None
        return None

    def __enter__(self):
        import threading
        if self.path is None:
            return self
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                v = self._read()
                if v is not None:
                    self.samples.append(v)
                self._stop.wait(self.period)

        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        return False

    def stats(self):
        if not self.samples:
            return None
        a = np.array(self.samples, dtype=np.float64)
        return {"median": float(np.median(a)), "min": float(a.min()), "max": float(a.max()),
                "samples": int(a.size), "source": "pp_dpm_sclk (current level), sampled every "
                f"{self.period * 1e3:.0f} ms during the event-bracketed runs"}


def timed_steps(torch, stream, step, K, Wm, samples=SAMPLES):
    """Wm untimed steps, then K timed steps (wall clock between two
    synchronizes, no events inside), then max(samples, K) more runs, each
    bracketed by HIP events on the run's stream (step(i, (ev0, ev1))), with the
    engine clock sampled meanwhile. Returns (wall ms per step, run ms of every
    bracketed run, clock stats)."""
    for i in range(Wm):
        step(i, None)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(Wm + i, None)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / K
    n = max(samples, K)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n)]
    with ClockSampler() as cs:
        for i in range(n):
            step(Wm + K + i, ev[i])
        torch.cuda.synchronize()
    return wall, np.array([a.elapsed_time(b) for a, b in ev]), cs.stats()


def replicas(t, torch, total_bytes):
    n = max(2, math.ceil(FLUSH_BYTES / max(total_bytes, 1)))
    return [t] + [t.clone() for _ in range(n - 1)], n


def plan_time_us(fn, n=50) -> float:
    t0 = time.perf_counter()
    for _ in range(n):
        fn()
    return (time.perf_counter() - t0) / n * 1e6


# ----------------------------------------------------------------------------
# decode (single, batch, skewed)
# ----------------------------------------------------------------------------
def bench_decode(abp, wl, torch, dev, w, K, Wm, workers=0, graph=False) -> dict:
    kv = w.kv
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float16
    by = decode_bytes(w)
    k0 = wl.to_torch(kv.k_pages, kv.dtype, dev)
    v0 = wl.to_torch(kv.v_pages, kv.dtype, dev)
    ks, copies = replicas(k0, torch, k0.nbytes + v0.nbytes)
    vs, _ = replicas(v0, torch, k0.nbytes + v0.nbytes)
    q = wl.to_torch(w.q, w.dtype, dev)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    indptr, indices, lpl = i32(kv.kv_indptr), i32(kv.kv_indices), i32(kv.kv_last_page_len)
    fp8 = kv.dtype == "fp8_e4m3"
    params = abp.make_params(w.num_qo_heads, w.num_kv_heads, w.head_dim, kv.page_size, dt,
                             kv_fp8=fp8, k_scale=w.k_scale, v_scale=w.v_scale)
    dec = abp.BatchDecode(params, max_batch=w.batch, num_workers=workers, device=dev)
    o = torch.empty(q.shape, dtype=dt, device=dev)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step(i, evs):
        dec.plan(kv.kv_indptr, kv.kv_last_page_len, stream=stream)
        if evs:
            evs[0].record(stream)
        dec.run(q, ks[i % copies], vs[i % copies], indptr, indices, lpl, o=o, lse=lse,
                stream=stream)
        if evs:
            evs[1].record(stream)

    wall, run_ms, clk = timed_steps(torch, stream, step, K, Wm)
    graph_leg = None
    if graph:
        # the same steps with run() captured once per K/V copy in a hipGraph and
        # replayed after each step's plan (the plan and its upload stay outside
        # the graph; the grid and the workspace are fixed, so a replay runs the
        # current plan)
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        graphs = []
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    dec.run(q, ks[c], vs[c], indptr, indices, lpl, o=o, lse=lse, stream=side)
            graphs.append(g)
        torch.cuda.synchronize()

        def gstep(i, evs):
            dec.plan(kv.kv_indptr, kv.kv_last_page_len, stream=stream)
            if evs:
                evs[0].record(stream)
            graphs[i % copies].replay()
            if evs:
                evs[1].record(stream)

        gwall, grun_ms, _ = timed_steps(torch, stream, gstep, K, Wm)
        torch.cuda.synchronize()
        graph_leg = {"step_TBps": round(by / (gwall * 1e-3) / 1e12, 4),
                     "ms_per_step": round(gwall, 5),
                     "run_TBps": round(by / (float(grun_ms.mean()) * 1e-3) / 1e12, 4),
                     "run": _stats_ms(grun_ms)}
    plan = dec.plan_struct
    hws = np.zeros(dec.host_ws.numel(), np.uint8)
    plan_us = plan_time_us(lambda: abp.abp_plan_host(
        abp.ABP_KIND_DECODE, params, w.batch, None, kv.kv_indptr, kv.kv_last_page_len, w.batch,
        0, plan.num_workers, hws))
    torch.cuda.synchronize()
    avg = float(run_ms.mean())
    return {
        "workload": w.name,
        "step_TBps": round(by / (wall * 1e-3) / 1e12, 4),
        "ms_per_step": round(wall, 5),
        "run_TBps": round(by / (avg * 1e-3) / 1e12, 4),
        "run": _stats_ms(run_ms),
        "clock_mhz": clk,
        "algorithmic_bytes": by,
        "plan_host_us": round(plan_us, 2),
        "batch": w.batch,
        "kv_tokens": int(kv.kv_len.sum()),
        "page_size": kv.page_size,
        "num_qo_heads": w.num_qo_heads,
        "num_kv_heads": w.num_kv_heads,
        "dtype": w.dtype,
        "kv_dtype": kv.dtype,
        "workers": plan.num_workers,
        "segments": plan.num_segments,
        "merged_tiles": plan.num_merges,
        "kv_pool_copies": copies,
        **({"graph_replay": graph_leg} if graph_leg else {}),
    }


# ----------------------------------------------------------------------------
# causal append
# ----------------------------------------------------------------------------
def bench_append(abp, wl, torch, dev, K, Wm, workers=0) -> dict:
    w = wl.ragged_append_causal()
    kv = w.kv
    flops = append_flops(w)
    q = wl.to_torch(w.q, w.dtype, dev)
    k0 = wl.to_torch(kv.k_pages, w.dtype, dev)
    v0 = wl.to_torch(kv.v_pages, w.dtype, dev)
    ks, copies = replicas(k0, torch, k0.nbytes + v0.nbytes)
    vs, _ = replicas(v0, torch, k0.nbytes + v0.nbytes)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    qo, indptr, indices, lpl = i32(w.qo_indptr), i32(kv.kv_indptr), i32(kv.kv_indices), \
        i32(kv.kv_last_page_len)
    params = abp.make_params(w.num_qo_heads, w.num_kv_heads, w.head_dim, kv.page_size,
                             torch.bfloat16, causal=True)
    app = abp.BatchAppend(params, max_batch=w.batch, max_qo_tokens=int(w.qo_indptr[-1]),
                          num_workers=workers, device=dev)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream(dev)

    def step(i, evs):
        app.plan(w.qo_indptr, kv.kv_indptr, kv.kv_last_page_len, stream=s)
        if evs:
            evs[0].record(s)
        app.run(q, ks[i % copies], vs[i % copies], qo, indptr, indices, lpl, o=o, lse=lse,
                stream=s)
        if evs:
            evs[1].record(s)

    wall, run_ms, clk = timed_steps(torch, s, step, K, Wm)
    hws = np.zeros(app.host_ws.numel(), np.uint8)
    nq = int(w.qo_indptr[-1])
    plan_us = plan_time_us(lambda: abp.abp_plan_host(
        abp.ABP_KIND_APPEND, params, w.batch, w.qo_indptr, kv.kv_indptr, kv.kv_last_page_len,
        w.batch, nq, app.plan_struct.num_workers, hws))
    torch.cuda.synchronize()
    avg = float(run_ms.mean())
    tf = flops / (avg * 1e-3) / 1e12
    return {
        "workload": w.name,
        "value": round(tf, 2),
        "unit": "TFLOP/s",
        "step_TFLOPs": round(flops / (wall * 1e-3) / 1e12, 2),
        "ms_per_step": round(wall, 5),
        "causal_flop": flops,
        "run": _stats_ms(run_ms),
        "clock_mhz": clk,
        "plan_host_us": round(plan_us, 2),
        "qo_tokens": int(w.qo_indptr[-1]),
        "kv_tokens": int(kv.kv_len.sum()),
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "append_kernel (split tiles merged in-kernel)",
                     "avg_launch_us": round(avg * 1e3, 2)},
        "workers": app.plan_struct.num_workers,
        "segments": app.plan_struct.num_segments,
        "merged_tiles": app.plan_struct.num_merges,
        "kv_pool_copies": copies,
    }


# ----------------------------------------------------------------------------
# mixed batch: decode + append in one launch, against the two runs in turn
# ----------------------------------------------------------------------------
def bench_pod(abp, wl, torch, dev, K, Wm) -> dict:
    w = wl.pod_mixed()
    d, a = w.dec, w.app
    by = decode_bytes(d)
    flops = append_flops(a)
    k0 = wl.to_torch(d.kv.k_pages, d.dtype, dev)
    v0 = wl.to_torch(d.kv.v_pages, d.dtype, dev)
    ks, copies = replicas(k0, torch, k0.nbytes + v0.nbytes)
    vs, _ = replicas(v0, torch, k0.nbytes + v0.nbytes)
    i32 = lambda x: torch.from_numpy(np.ascontiguousarray(x, np.int32)).to(dev)
    qd, qa = wl.to_torch(d.q, d.dtype, dev), wl.to_torch(a.q, a.dtype, dev)
    d_ip, d_ix, d_lp = i32(d.kv.kv_indptr), i32(d.kv.kv_indices), i32(d.kv.kv_last_page_len)
    qo, a_ip, a_ix, a_lp = (i32(a.qo_indptr), i32(a.kv.kv_indptr), i32(a.kv.kv_indices),
                            i32(a.kv.kv_last_page_len))
    nd, na, nq = d.batch, len(a.kv.kv_indptr) - 1, int(a.qo_indptr[-1])
    pd = abp.make_params(32, 8, 128, 16, torch.bfloat16)
    pa = abp.make_params(32, 8, 128, 16, torch.bfloat16, causal=True)
    dec = abp.BatchDecode(pd, max_batch=nd, device=dev)
    app = abp.BatchAppend(pa, max_batch=na, max_qo_tokens=nq, device=dev)
    pod = abp.PodAttention(pa, nd, na, nq, device=dev)
    od, ld = torch.empty_like(qd), torch.empty(qd.shape[:2], dtype=torch.float32, device=dev)
    oa, la = torch.empty_like(qa), torch.empty(qa.shape[:2], dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream(dev)
    dec.plan(d.kv.kv_indptr, d.kv.kv_last_page_len, stream=s)
    app.plan(a.qo_indptr, a.kv.kv_indptr, a.kv.kv_last_page_len, stream=s)
    plan = pod.plan(d.kv.kv_indptr, d.kv.kv_last_page_len, a.qo_indptr, a.kv.kv_indptr,
                    a.kv.kv_last_page_len, stream=s)

    def seq(i, evs):
        if evs:
            evs[0].record(s)
        dec.run(qd, ks[i % copies], vs[i % copies], d_ip, d_ix, d_lp, o=od, lse=ld, stream=s)
        app.run(qa, ks[i % copies], vs[i % copies], qo, a_ip, a_ix, a_lp, o=oa, lse=la, stream=s)
        if evs:
            evs[1].record(s)

    def mixed(i, evs):
        if evs:
            evs[0].record(s)
        pod.run(qd, qa, ks[i % copies], vs[i % copies], d_ip, d_ix, d_lp, qo, a_ip, a_ix, a_lp,
                o_decode=od, lse_decode=ld, o_append=oa, lse_append=la, stream=s)
        if evs:
            evs[1].record(s)

    _, seq_ms, _ = timed_steps(torch, s, seq, K, Wm)
    wall, pod_ms, clk = timed_steps(torch, s, mixed, K, Wm)
    torch.cuda.synchronize()
    t_seq, t_pod = float(seq_ms.mean()), float(pod_ms.mean())
    return {
        "workload": w.name,
        "value": round(t_seq / t_pod, 4),
        "unit": "speedup over the decode run then the append run",
        "run": _stats_ms(pod_ms),
        "clock_mhz": clk,
        "sequential_run": _stats_ms(seq_ms),
        "ms_per_step": round(wall, 5),
        "decode_bytes": by,
        "append_causal_flop": flops,
        "decode_TBps_over_run": round(by / (t_pod * 1e-3) / 1e12, 4),
        "append_TFLOPs_over_run": round(flops / (t_pod * 1e-3) / 1e12, 2),
        # the decode part's HBM bytes bound the batch (at peak they take longer
        # than the append part's flop at the dense bf16 peak)
        "roofline": {"bound": "hbm", "achieved": round(by / (t_pod * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_TBS * 1e3, "unit": "GB/s",
                     "frac": round(by / (t_pod * 1e-3) / 1e12 / HBM_PEAK_TBS, 4),
                     "traffic": None,
                     "kernel": "pod_kernel + the two plan merges (one run; it also does the "
                               "append part's flop)",
                     "avg_launch_us": round(t_pod * 1e3, 2)},
        "split": {"groups": plan.num_groups, "decode": plan.decode.num_workers,
                  "append": plan.append.num_workers},
        "sequential_workers": {"decode": dec.plan_struct.num_workers,
                               "append": app.plan_struct.num_workers},
        "kv_pool_copies": copies,
    }


# ----------------------------------------------------------------------------
# cascade (shared prefix + suffixes, RoPE)
# ----------------------------------------------------------------------------
def bench_cascade(abp, wl, torch, dev, K, Wm, workers=0) -> dict:
    w = wl.cascade_rope()
    pre, kv = w.prefix, w.kv
    by = cascade_bytes(w)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    tot = pre.k_pages.nbytes * 2 + kv.k_pages.nbytes * 2
    pk, copies = replicas(wl.to_torch(pre.k_pages, w.dtype, dev), torch, tot)
    pv, _ = replicas(wl.to_torch(pre.v_pages, w.dtype, dev), torch, tot)
    sk, _ = replicas(wl.to_torch(kv.k_pages, w.dtype, dev), torch, tot)
    sv, _ = replicas(wl.to_torch(kv.v_pages, w.dtype, dev), torch, tot)
    q = wl.to_torch(w.q, w.dtype, dev)
    cas = abp.CascadeDecode(w.num_qo_heads, w.num_kv_heads, w.head_dim, pre.page_size,
                            kv.page_size, torch.bfloat16, max_batch=w.batch,
                            rope_theta=w.rope_theta, num_workers=workers, device=dev)
    pqo = i32([0, w.batch])
    p_ind, p_idx, p_lpl = i32(pre.kv_indptr), i32(pre.kv_indices), i32(pre.kv_last_page_len)
    s_ind, s_idx, s_lpl = i32(kv.kv_indptr), i32(kv.kv_indices), i32(kv.kv_last_page_len)
    qpos, kvoff = i32(w.q_pos), i32(w.kv_pos_offset)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    bufs = cas.buffers(q)
    s = torch.cuda.current_stream(dev)

    def plan():
        cas.plan(w.batch, pre.kv_indptr, pre.kv_last_page_len, kv.kv_indptr,
                 kv.kv_last_page_len, stream=s)

    def step(i, evs):
        plan()
        if evs:
            evs[0].record(s)
        c = i % copies
        cas.run(q, pk[c], pv[c], pqo, p_ind, p_idx, p_lpl, sk[c], sv[c], s_ind, s_idx, s_lpl,
                q_pos=qpos, kv_pos_offset=kvoff, o=o, lse=lse, stream=s, bufs=bufs)
        if evs:
            evs[1].record(s)

    wall, run_ms, clk = timed_steps(torch, s, step, K, Wm)
    torch.cuda.synchronize()
    avg = float(run_ms.mean())
    return {
        "workload": w.name,
        "clock_mhz": clk,
        "step_TBps": round(by / (wall * 1e-3) / 1e12, 4),
        "ms_per_step": round(wall, 5),
        "run_TBps": round(by / (avg * 1e-3) / 1e12, 4),
        "run": _stats_ms(run_ms),
        "algorithmic_bytes": by,
        "batch": w.batch,
        "prefix_tokens": int(pre.kv_len.sum()),
        "suffix_tokens": int(kv.kv_len.sum()),
        "rope_theta": w.rope_theta,
        "launches": "prefix append (RoPE) + suffix decode (RoPE) + one merge of both levels' states",
        "kv_pool_copies": copies,
    }


# ----------------------------------------------------------------------------
# the pages' comparisons on this chip (cascade workload): RoPE fused at load
# against a separate rotation pass, and the cascade against a flat page table
# ----------------------------------------------------------------------------
def _rope_tables(torch, dev, pos, theta, d=128):
    """cos / sin of pos * theta^(-2j/d), j < d/2, for a position array (fp32;
    the separate pass's own inputs, built once outside the timed region)."""
    f = torch.tensor(theta ** (-np.arange(d // 2, dtype=np.float64) * 2.0 / d),
                     dtype=torch.float64, device=dev)
    ang = torch.from_numpy(np.asarray(pos, np.float64)).to(dev)[..., None] * f
    return torch.cos(ang).float(), torch.sin(ang).float()


def _slot_positions(kv, offset):
    """Position of every slot of a pool [num_pages, page_size] under its page
    table: request b's logical token t sits at offset[b] + t (unused slots: 0)."""
    pos = np.zeros((kv.num_pages, kv.page_size), np.int64)
    for b in range(len(kv.kv_indptr) - 1):
        pages = kv.kv_indices[kv.kv_indptr[b]:kv.kv_indptr[b + 1]]
        for i, pg in enumerate(pages):
            pos[pg] = offset[b] + i * kv.page_size + np.arange(kv.page_size)
    return pos


def bench_cascade_separate_rope(abp, wl, torch, dev, K, Wm, fused_us) -> dict:
    """Rotate-then-attend: a separate pass (PyTorch elementwise ops) writes
    rotated q and rotated K pools, then the cascade runs without RoPE on them."""
    w = wl.cascade_rope()
    pre, kv = w.prefix, w.kv
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    theta = w.rope_theta
    tot = pre.k_pages.nbytes * 2 + kv.k_pages.nbytes * 2
    pk, copies = replicas(wl.to_torch(pre.k_pages, w.dtype, dev), torch, tot)
    pv, _ = replicas(wl.to_torch(pre.v_pages, w.dtype, dev), torch, tot)
    sk, _ = replicas(wl.to_torch(kv.k_pages, w.dtype, dev), torch, tot)
    sv, _ = replicas(wl.to_torch(kv.v_pages, w.dtype, dev), torch, tot)
    q = wl.to_torch(w.q, w.dtype, dev)
    pc, ps = _rope_tables(torch, dev, _slot_positions(pre, [0]), theta)
    sc, ss = _rope_tables(torch, dev, _slot_positions(kv, w.kv_pos_offset), theta)
    qc, qs = _rope_tables(torch, dev, w.q_pos, theta)
    pre_rot = torch.empty_like(pk[0])
    suf_rot = torch.empty_like(sk[0])
    q_rot = torch.empty_like(q)

    def rotate(x, c, sn, out):
        # x [..., H, 128]: rotate-half pairs (j, j + 64); c / sn [..., 64] broadcast over H
        xf = x.float()
        a, b = xf[..., :64], xf[..., 64:]
        c, sn = c.unsqueeze(-2), sn.unsqueeze(-2)
        out[..., :64] = (a * c - b * sn).to(out.dtype)
        out[..., 64:] = (b * c + a * sn).to(out.dtype)

    cas = abp.CascadeDecode(w.num_qo_heads, w.num_kv_heads, w.head_dim, pre.page_size,
                            kv.page_size, torch.bfloat16, max_batch=w.batch, rope_theta=0.0,
                            device=dev)
    pqo = i32([0, w.batch])
    p_ind, p_idx, p_lpl = i32(pre.kv_indptr), i32(pre.kv_indices), i32(pre.kv_last_page_len)
    s_ind, s_idx, s_lpl = i32(kv.kv_indptr), i32(kv.kv_indices), i32(kv.kv_last_page_len)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    bufs = cas.buffers(q)
    s = torch.cuda.current_stream(dev)

    def step(i, evs):
        cas.plan(w.batch, pre.kv_indptr, pre.kv_last_page_len, kv.kv_indptr,
                 kv.kv_last_page_len, stream=s)
        if evs:
            evs[0].record(s)
        c = i % copies
        rotate(q, qc, qs, q_rot)
        rotate(pk[c], pc, ps, pre_rot)
        rotate(sk[c], sc, ss, suf_rot)
        cas.run(q_rot, pre_rot, pv[c], pqo, p_ind, p_idx, p_lpl, suf_rot, sv[c], s_ind, s_idx,
                s_lpl, o=o, lse=lse, stream=s, bufs=bufs)
        if evs:
            evs[1].record(s)

    wall, run_ms, clk = timed_steps(torch, s, step, K, Wm)
    avg_us = float(run_ms.mean()) * 1e3
    return {
        "what": "rotate q and both K pools with PyTorch elementwise ops (fp32 math, bf16 "
                "results, 12 launches), then the cascade without RoPE; against the cascade "
                "with RoPE fused at load",
        "run": _stats_ms(run_ms),
        "clock_mhz": clk,
        "fused_run_avg_us": round(fused_us, 2),
        "value": round(avg_us / fused_us, 3),
        "unit": "separate-pass run time / fused run time",
        "note": "the rotated K pools are rounded to bf16, which costs the separate pass "
                "accuracy the fused path keeps (its scores use fp32 / hi+lo operands)",
    }


def bench_flat_decode(abp, wl, torch, dev, K, Wm, cascade_us) -> dict:
    """The cascade workload as one flat page table of 16-token pages: every
    request lists the shared prefix's pages, then its own, so each request
    reads the prefix again; RoPE decode over prefix || suffix."""
    w = wl.cascade_rope()
    pre, kv = w.prefix, w.kv
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    P = kv.page_size
    pl = int(pre.kv_len[0])
    # the prefix's keys in logical order, cut into pages of P (shared by every request)
    order = pre.kv_indices[pre.kv_indptr[0]:pre.kv_indptr[1]]
    klog = pre.k_pages[order].reshape(-1, w.num_kv_heads, w.head_dim)[:pl]
    vlog = pre.v_pages[order].reshape(-1, w.num_kv_heads, w.head_dim)[:pl]
    npre = -(-pl // P)
    pad = npre * P - pl
    kpre = np.concatenate([klog, np.zeros((pad,) + klog.shape[1:], klog.dtype)]).reshape(
        npre, P, w.num_kv_heads, w.head_dim)
    vpre = np.concatenate([vlog, np.zeros((pad,) + vlog.shape[1:], vlog.dtype)]).reshape(
        npre, P, w.num_kv_heads, w.head_dim)
    assert pad == 0, "the prefix fills whole 16-token pages"
    kflat = np.concatenate([kpre, kv.k_pages])
    vflat = np.concatenate([vpre, kv.v_pages])
    B = w.batch
    lens = np.diff(kv.kv_indptr)
    indptr = np.concatenate([[0], np.cumsum(lens + npre)]).astype(np.int32)
    idx = np.concatenate([np.concatenate([np.arange(npre),
                                          kv.kv_indices[kv.kv_indptr[b]:kv.kv_indptr[b + 1]] + npre])
                          for b in range(B)]).astype(np.int32)
    lpl = kv.kv_last_page_len
    k0, v0 = wl.to_torch(kflat, w.dtype, dev), wl.to_torch(vflat, w.dtype, dev)
    ks, copies = replicas(k0, torch, k0.nbytes + v0.nbytes)
    vs, _ = replicas(v0, torch, k0.nbytes + v0.nbytes)
    q = wl.to_torch(w.q, w.dtype, dev)
    params = abp.make_params(w.num_qo_heads, w.num_kv_heads, w.head_dim, P, torch.bfloat16,
                             rope_theta=w.rope_theta)
    dec = abp.BatchDecode(params, max_batch=B, device=dev)
    d_ind, d_idx, d_lpl = i32(indptr), i32(idx), i32(lpl)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream(dev)

    def step(i, evs):
        dec.plan(indptr, lpl, stream=s)
        if evs:
            evs[0].record(s)
        c = i % copies
        # default positions: key t at t, the query on the last key (= the cascade's)
        dec.run(q, ks[c], vs[c], d_ind, d_idx, d_lpl, o=o, lse=lse, stream=s)
        if evs:
            evs[1].record(s)

    wall, run_ms, clk = timed_steps(torch, s, step, K, Wm)
    avg_us = float(run_ms.mean()) * 1e3
    logical = (B * pl + int(kv.kv_len.sum())) * w.num_kv_heads * w.head_dim * 2 * 2
    return {
        "what": "one flat page table (pages of 16): each request lists the prefix's pages and "
                "then its own; RoPE batch decode; against the cascade",
        "run": _stats_ms(run_ms),
        "clock_mhz": clk,
        "logical_kv_bytes": logical,
        "cascade_run_avg_us": round(cascade_us, 2),
        "value": round(avg_us / cascade_us, 3),
        "unit": "flat run time / cascade run time",
    }


# ----------------------------------------------------------------------------
# block-sparse attention (MFMA) and page append (HBM copy)
# ----------------------------------------------------------------------------
def bsr_flops(w, rows=None) -> float:
    """4 * d * Hq per (query, key) pair the mask lets through."""
    nrb = len(w.indptr) - 1
    cnt = np.diff(w.indptr).astype(np.int64)
    if rows is None:
        per_block = np.minimum((np.arange(nrb) + 1) * w.R, w.M) - np.arange(nrb) * w.R
        pairs = int((per_block * cnt).sum()) * w.C
    else:
        pairs = int(sum(int(cnt[r // w.R]) for r in rows)) * w.C
    return 4.0 * w.head_dim * w.num_qo_heads * float(pairs)


def bench_bsr(abp, wl, torch, dev, K, Wm) -> dict:
    w = wl.bsr_sparse()
    flops = bsr_flops(w)
    q = wl.to_torch(w.q, w.dtype, dev)
    k0 = wl.to_torch(w.k, w.dtype, dev)
    v0 = wl.to_torch(w.v, w.dtype, dev)
    ks, copies = replicas(k0, torch, k0.nbytes + v0.nbytes)
    vs, _ = replicas(v0, torch, k0.nbytes + v0.nbytes)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    ip, idx = i32(w.indptr), i32(w.indices)
    params = abp.make_params(w.num_qo_heads, w.num_kv_heads, w.head_dim, w.C, torch.bfloat16)
    nrb = len(w.indptr) - 1
    bsr = abp.BlockSparseAttention(params, max_row_blocks=nrb, max_M=w.M, device=dev)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream(dev)

    def step(i, evs):
        bsr.plan(w.M, w.N, w.R, w.indptr, stream=s)
        if evs:
            evs[0].record(s)
        bsr.run(q, ks[i % copies], vs[i % copies], ip, idx, o=o, lse=lse, stream=s)
        if evs:
            evs[1].record(s)

    wall, run_ms, clk = timed_steps(torch, s, step, K, Wm)
    torch.cuda.synchronize()
    avg = float(run_ms.mean())
    tf = flops / (avg * 1e-3) / 1e12
    nnz = int(w.indptr[-1])
    return {
        "workload": w.name,
        "value": round(tf, 2),
        "unit": "TFLOP/s",
        "step_TFLOPs": round(flops / (wall * 1e-3) / 1e12, 2),
        "ms_per_step": round(wall, 5),
        "mask_flop": flops,
        "density": round(nnz / (nrb * (w.N // w.C)), 4),
        "run": _stats_ms(run_ms),
        "clock_mhz": clk,
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                     "traffic": None, "kernel": "append_kernel over BSR row blocks (+ merge)",
                     "avg_launch_us": round(avg * 1e3, 2)},
        "workers": bsr.plan_struct.num_workers,
        "segments": bsr.plan_struct.num_segments,
        "kv_copies": copies,
    }


def page_append_bytes(w) -> int:
    """Each new K/V row read once and written once, plus append_indptr, the page
    table entries read (kv_indptr, last_page_len, one index per row)."""
    kv = w.kv
    row = kv.num_kv_heads * kv.head_dim * 2
    B = len(w.append_indptr) - 1
    return 2 * 2 * w.nnz * row + (B + 1) * 4 + (B + 1) * 4 + B * 4 + w.nnz * 4


def bench_page_append(abp, wl, torch, dev, K, Wm) -> dict:
    w = wl.ragged_page_append()
    kv = w.kv
    by = page_append_bytes(w)
    kn0 = wl.to_torch(w.k_new, kv.dtype, dev)
    vn0 = wl.to_torch(w.v_new, kv.dtype, dev)
    kp0 = wl.to_torch(kv.k_pages, kv.dtype, dev)
    vp0 = wl.to_torch(kv.v_pages, kv.dtype, dev)
    tot = kn0.nbytes * 2 + kp0.nbytes * 2
    kns, copies = replicas(kn0, torch, tot)
    vns, _ = replicas(vn0, torch, tot)
    kps, _ = replicas(kp0, torch, tot)
    vps, _ = replicas(vp0, torch, tot)
    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(dev)
    ai, ip, idx, lpl = i32(w.append_indptr), i32(kv.kv_indptr), i32(kv.kv_indices), \
        i32(kv.kv_last_page_len)
    s = torch.cuda.current_stream(dev)
    # a launch is ~16 us: one event pair per group of GROUP back-to-back launches,
    # so the events' own idle time is spread over the group
    GROUP = 8

    def step(i, evs):
        if evs:
            evs[0].record(s)
        for j in range(GROUP):
            c = (i * GROUP + j) % copies
            abp.append_paged_kv_cache(kns[c], vns[c], ai, kps[c], vps[c], ip, idx, lpl, stream=s)
        if evs:
            evs[1].record(s)

    wall, run_ms, clk = timed_steps(torch, s, step, max(1, K // GROUP), max(1, Wm // GROUP))
    torch.cuda.synchronize()
    wall /= GROUP
    run_ms = run_ms / GROUP
    avg = float(run_ms.mean())
    gbs = by / (avg * 1e-3) / 1e9
    tr = recorded_traffic(PAGE_APPEND_TRAFFIC_FILE, PAGE_APPEND_SOURCES)
    return {
        "workload": w.name,
        "value": round(gbs / 1e3, 4),
        "unit": "TB/s",
        "ms_per_step": round(wall, 5),
        "algorithmic_bytes": by,
        "new_tokens": w.nnz,
        "run": _stats_ms(run_ms),
        "clock_mhz": clk,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_TBS * 1e3,
                     "unit": "GB/s", "frac": round(gbs / (HBM_PEAK_TBS * 1e3), 4),
                     "traffic": tr["traffic_bytes_per_run"] if tr else None,
                     "kernel": "page_append_kernel",
                     "avg_launch_us": round(avg * 1e3, 2)},
        "timing": f"HIP events around groups of {GROUP} back-to-back launches",
        "copies": copies,
    }


# ----------------------------------------------------------------------------
# plain copy (context and counter calibration)
# ----------------------------------------------------------------------------
def bench_copy(torch, dev, K, Wm, nbytes=2 ** 30) -> dict:
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=dev).normal_()
    b = torch.empty_like(a)
    s = torch.cuda.current_stream(dev)

    def step(i, evs):
        if evs:
            evs[0].record(s)
        b.copy_(a)
        if evs:
            evs[1].record(s)

    _, ms, _ = timed_steps(torch, s, step, K, Wm, samples=K)
    avg = float(ms.mean())
    return {"bytes_read": nbytes, "bytes_written": nbytes,
            "read_plus_write_TBps": round(2 * nbytes / (avg * 1e-3) / 1e12, 4),
            "run": _stats_ms(ms)}


# ----------------------------------------------------------------------------
# CPU baseline: the oracle, bounded sample
# ----------------------------------------------------------------------------
def _cpu_info():
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return model, len(os.sched_getaffinity(0))


def cpu_baseline_decode(w, budget_s: float = 12.0) -> dict:
    """The fp64 oracle over whole requests of the batch, repeated passes, until
    about budget_s of CPU time (one BLAS thread)."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as ora
    t_used, by, n_req = 0.0, 0, 0
    with threadpool_limits(limits=1):
        while t_used < budget_s:
            for b in range(w.batch):
                t0 = time.perf_counter()
                ora.decode_workload(w, batch_ids=[b])
                t_used += time.perf_counter() - t0
                by += decode_bytes(w, [b])
                n_req += 1
                if t_used >= budget_s:
                    break
    model, avail = _cpu_info()
    return {"value": round(by / t_used / 1e12, 6), "unit": "TB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n_req} request evaluations ({n_req / w.batch:.2f} passes over the "
                      f"{w.batch}-request batch, {by / 1e9:.2f} GB algorithmic) in "
                      f"{t_used:.1f} s; fp64 NumPy, 1 BLAS thread",
            "host_cpu": model, "host_cores_available": avail}


def cpu_baseline_append(w, budget_s: float = 8.0) -> dict:
    from threadpoolctl import threadpool_limits

    from oracle import attention as ora
    rng = np.random.Generator(np.random.PCG64(7))
    qo = np.diff(w.qo_indptr)
    done, t_used = [], 0.0
    with threadpool_limits(limits=1):
        while t_used < budget_s:
            b = int(rng.integers(0, w.batch))
            n = min(32, int(qo[b]))
            i0 = int(w.qo_indptr[b]) + int(rng.integers(0, int(qo[b]) - n + 1))
            ids = list(range(i0, i0 + n))
            t0 = time.perf_counter()
            ora.append_workload(w, token_ids=ids)
            t_used += time.perf_counter() - t0
            done += ids
    fl = append_flops(w, done)
    model, avail = _cpu_info()
    return {"value": round(fl / t_used / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{len(done)} of {int(w.qo_indptr[-1])} query tokens (runs of 32 at random "
                      f"places, all heads; "
                      f"{fl / 1e9:.1f} GFLOP visible) in {t_used:.1f} s; fp64 NumPy, 1 BLAS "
                      f"thread", "host_cpu": model, "host_cores_available": avail}


def cpu_baseline_pod(w, budget_s: float = 3.0) -> dict:
    """The oracle on the mixed batch: its decode and append rates, each measured
    as in the decode and append baselines on that part, give the time of the
    whole batch."""
    d = cpu_baseline_decode(w.dec, budget_s)
    a = cpu_baseline_append(w.app, budget_s)
    t = decode_bytes(w.dec) / (d["value"] * 1e12) + append_flops(w.app) / (a["value"] * 1e12)
    return {"value": round(t, 3), "unit": "s per mixed batch", "cores": 1, "kind": "oracle",
            "sample": f"decode part: {d['sample']}; append part: {a['sample']}; the batch's "
                      f"decode bytes and append flop at those rates",
            "host_cpu": d["host_cpu"], "host_cores_available": d["host_cores_available"]}


def cpu_baseline_bsr(w, budget_s: float = 6.0) -> dict:
    """The fp64 oracle on runs of 8 query rows at random places (all heads)."""
    from threadpoolctl import threadpool_limits

    from oracle import attention as ora
    rng = np.random.Generator(np.random.PCG64(8))
    done, t_used = [], 0.0
    with threadpool_limits(limits=1):
        while t_used < budget_s:
            r0 = int(rng.integers(0, w.M - 8))
            rows = list(range(r0, r0 + 8))
            t0 = time.perf_counter()
            ora.bsr_attention(w.q, w.k, w.v, w.R, w.C, w.indptr, w.indices, w.dtype,
                              w.num_kv_heads, rows=rows)
            t_used += time.perf_counter() - t0
            done += rows
    fl = bsr_flops(w, done)
    model, avail = _cpu_info()
    return {"value": round(fl / t_used / 1e12, 6), "unit": "TFLOP/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{len(done)} of {w.M} query rows (runs of 8, all heads; {fl / 1e9:.1f} "
                      f"GFLOP in the mask) in {t_used:.1f} s; fp64 NumPy, 1 BLAS thread",
            "host_cpu": model, "host_cores_available": avail}


def cpu_baseline_page_append(w, budget_s: float = 4.0) -> dict:
    """The oracle's page append over the whole workload, repeated."""
    from oracle import attention as ora
    kv = w.kv
    n, t_used = 0, 0.0
    while t_used < budget_s:
        t0 = time.perf_counter()
        ora.append_paged_kv(w.k_new, w.v_new, w.append_indptr, kv.k_pages, kv.v_pages,
                            kv.kv_indptr, kv.kv_indices, kv.kv_last_page_len, kv.page_size)
        t_used += time.perf_counter() - t0
        n += 1
    model, avail = _cpu_info()
    return {"value": round(n * page_append_bytes(w) / t_used / 1e12, 6), "unit": "TB/s",
            "cores": 1, "kind": "oracle",
            "sample": f"{n} passes over all {w.nnz} new rows (each pass copies both pools) in "
                      f"{t_used:.1f} s; NumPy, one thread",
            "host_cpu": model, "host_cores_available": avail}


# ----------------------------------------------------------------------------
def comparisons(abp, wl, torch, dev, K, configs) -> dict:
    """The pages' three comparisons, measured here as ratios (> 1: the method wins):
    the Stream-K split against one worker per tile on skewed lengths (paper
    summary, 动态负载均衡调度 / 性能提升), RoPE fused at load against a
    separate rotation pass (可定制的注意力模板 / 性能提升), and the cascade
    against a flat page table that reads the prefix once per request
    (统一的 KV 缓存存储格式 / 高级功能)."""
    sk = configs["skewed_decode"]
    ns = bench_decode(abp, wl, torch, dev, wl.skewed_decode_gqa(), K, 5,
                      abp.ABP_WORKERS_PER_TILE)
    cas_us = configs["cascade_rope"]["run"]["avg_us"]
    sep = bench_cascade_separate_rope(abp, wl, torch, dev, K, 5, cas_us)
    flat = bench_flat_decode(abp, wl, torch, dev, K, 5, cas_us)
    return {
        "load_balance_skewed": {
            "value": round(ns["run"]["avg_us"] / sk["run"]["avg_us"], 3),
            "unit": "one-worker-per-tile run time / Stream-K run time",
            "no_split_run": ns["run"], "no_split_workers": ns["workers"],
            "stream_k_run": sk["run"], "stream_k_workers": sk["workers"],
            "clock_mhz": ns["clock_mhz"],
        },
        "rope_fused_vs_separate": sep,
        "cascade_vs_flat": flat,
    }


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workers", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-append", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the single, skewed and cascade workloads")
    ap.add_argument("--part", default="all",
                    choices=["all", "decode", "append", "single", "skewed", "cascade", "copy",
                             "bsr", "page_append", "fp8_decode", "g8_decode", "pod",
                             "comparisons"],
                    help="one workload alone (profiling); 'all' is the benchmark line")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (each GPU "
              "would run its own share of requests or kv heads with no exchange); use --gpus 1",
              file=sys.stderr)
        return 2

    import torch

    import attention_bsr_paged_amd as abp
    from attention_bsr_paged_amd import workloads as wl

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    abp.load_library()
    K, Wm = args.steps, args.warmup
    part = args.part
    if part == "append":
        print(json.dumps(bench_append(abp, wl, torch, dev, K, Wm, args.workers)), flush=True)
        return 0
    if part == "copy":
        print(json.dumps(bench_copy(torch, dev, K, Wm)), flush=True)
        return 0
    if part == "cascade":
        print(json.dumps(bench_cascade(abp, wl, torch, dev, K, Wm, args.workers)), flush=True)
        return 0
    if part == "bsr":
        print(json.dumps(bench_bsr(abp, wl, torch, dev, K, Wm)), flush=True)
        return 0
    if part == "page_append":
        print(json.dumps(bench_page_append(abp, wl, torch, dev, K, Wm)), flush=True)
        return 0
    if part == "pod":
        print(json.dumps(bench_pod(abp, wl, torch, dev, K, Wm)), flush=True)
        return 0
    if part == "comparisons":
        cfg = {"skewed_decode": bench_decode(abp, wl, torch, dev, wl.skewed_decode_gqa(), K, Wm),
               "cascade_rope": bench_cascade(abp, wl, torch, dev, K, Wm)}
        print(json.dumps(comparisons(abp, wl, torch, dev, K, cfg)), flush=True)
        return 0
    if part in ("single", "skewed", "fp8_decode", "g8_decode"):
        w = {"single": wl.single_decode_mha, "skewed": wl.skewed_decode_gqa,
             "fp8_decode": wl.batch_decode_fp8,
             "g8_decode": lambda: wl.batch_decode_gqa(num_qo_heads=64)}[part]()
        print(json.dumps(bench_decode(abp, wl, torch, dev, w, K, Wm, args.workers)), flush=True)
        return 0

    # --------------------------------------------------- batch decode (the line)
    w = wl.batch_decode_gqa()
    d = bench_decode(abp, wl, torch, dev, w, K, Wm, args.workers, graph=True)
    by = d["algorithmic_bytes"]
    avg_s = d["run"]["avg_us"] * 1e-6
    achieved = by / avg_s / 1e9
    tr = recorded_traffic()
    out = {
        "metric": "paged-decode achieved HBM TB/s (% of peak) + causal-append TFLOPS, bf16 GQA",
        "value": d["step_TBps"],
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": d["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) values rounded to bf16, uniform kv_len, shuffled "
                "page pool",
        "config": {
            "workload": "batch paged decode: 64 requests, kv_len U{512..4096}, GQA 32/8, "
                        "head_dim 128, page_size 16, bf16",
            "batch": d["batch"],
            "num_qo_heads": d["num_qo_heads"],
            "num_kv_heads": d["num_kv_heads"],
            "head_dim": 128,
            "page_size": d["page_size"],
            "kv_tokens": d["kv_tokens"],
            "algorithmic_bytes": by,
            "workers": d["workers"],
            "segments": d["segments"],
            "merged_tiles": d["merged_tiles"],
            "kv_pool_copies": d["kv_pool_copies"],
            "parallelism": "single GPU",
        },
        "pct_of_hbm_peak": round(100 * d["step_TBps"] / HBM_PEAK_TBS, 2),
        # the same steps with run() replayed from a hipGraph (reported beside
        # `value`, which times the eager launches)
        "graph_replay": d.get("graph_replay"),
        "clock_mhz": d["clock_mhz"],
        "plan_host_us": d["plan_host_us"],
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_TBS * 1e3,
            "unit": "GB/s",
            "frac": round(achieved / (HBM_PEAK_TBS * 1e3), 4),
            "traffic": tr["traffic_bytes_per_run"] if tr else None,
            "kernel": "decode run: decode_mfma_kernel + plan_merge_kernel (one run() call)",
            "avg_launch_us": d["run"]["avg_us"],
            "median_us": d["run"]["median_us"],
            "p10_us": d["run"]["p10_us"],
            "p90_us": d["run"]["p90_us"],
        },
    }
    if part == "all" and not args.no_append:
        out["append"] = bench_append(abp, wl, torch, dev, max(20, K // 4), 5)
    if part == "all" and not args.no_configs:
        Kc = max(20, K // 2)
        out["configs"] = {
            "single_decode": bench_decode(abp, wl, torch, dev, wl.single_decode_mha(), Kc, 5),
            "skewed_decode": bench_decode(abp, wl, torch, dev, wl.skewed_decode_gqa(), Kc, 5),
            "cascade_rope": bench_cascade(abp, wl, torch, dev, Kc, 5),
        }
        out["comparisons"] = comparisons(abp, wl, torch, dev, Kc, out["configs"])
        out["next"] = {
            "bsr_sparse": bench_bsr(abp, wl, torch, dev, Kc, 5),
            "page_append": bench_page_append(abp, wl, torch, dev, Kc, 5),
            "fp8_batch_decode": bench_decode(abp, wl, torch, dev, wl.batch_decode_fp8(), Kc, 5),
            "pod_mixed": bench_pod(abp, wl, torch, dev, Kc, 5),
        }
        f8 = out["next"]["fp8_batch_decode"]
        f8["roofline"] = {"bound": "hbm", "achieved": round(f8["run_TBps"] * 1e3, 1),
                          "peak": HBM_PEAK_TBS * 1e3, "unit": "GB/s",
                          "frac": round(f8["run_TBps"] / HBM_PEAK_TBS, 4), "traffic": None,
                          "kernel": "decode run, e4m3 K/V (decode_mfma_fp8_kernel + plan_merge_kernel)",
                          "avg_launch_us": f8["run"]["avg_us"]}
        f8["kv_tokens_per_s"] = round(f8["kv_tokens"] / (f8["run"]["avg_us"] * 1e-6), 1)
        out["copy_context"] = bench_copy(torch, dev, 20, 3)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_decode(w)
        if "append" in out:
            out["append"]["cpu_baseline"] = cpu_baseline_append(wl.ragged_append_causal())
        if "next" in out:
            out["next"]["bsr_sparse"]["cpu_baseline"] = cpu_baseline_bsr(wl.bsr_sparse())
            out["next"]["page_append"]["cpu_baseline"] = \
                cpu_baseline_page_append(wl.ragged_page_append())
            out["next"]["fp8_batch_decode"]["cpu_baseline"] = \
                cpu_baseline_decode(wl.batch_decode_fp8(), budget_s=4.0)
            out["next"]["pod_mixed"]["cpu_baseline"] = cpu_baseline_pod(wl.pod_mixed())
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
