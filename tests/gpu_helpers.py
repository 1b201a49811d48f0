"""Shared helpers of the GPU tests: upload a workload, run it through the
binding (C ABI), and compare with the oracle to the parity bar."""
from __future__ import annotations

import sys

import numpy as np

import attention_bsr_paged_amd as abp
from attention_bsr_paged_amd import workloads as wl

# Parity bar: max-abs error of o (rounded to the storage type) and of lse
# (natural log, fp32) against the fp64 oracle.
O_TOL = {"fp16": 1e-2, "bf16": 2e-2}
LSE_TOL = 1e-3


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def torch_dtype(name):
    import torch
    return torch.bfloat16 if name == "bf16" else torch.float16


def upload_kv(kv, device="cuda"):
    import torch
    return dict(
        k=wl.to_torch(kv.k_pages, kv.dtype, device),
        v=wl.to_torch(kv.v_pages, kv.dtype, device),
        indptr=torch.from_numpy(kv.kv_indptr).to(device),
        indices=torch.from_numpy(kv.kv_indices).to(device),
        lpl=torch.from_numpy(kv.kv_last_page_len).to(device),
    )


def i32(a, device="cuda"):
    import torch
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(device)


def run_decode(w, num_workers=0, out_dtype=None, dev=None, return_runner=False):
    import torch
    kv = w.kv
    dev = dev or upload_kv(kv)
    q = wl.to_torch(w.q, w.dtype, "cuda")
    params = abp.make_params(w.num_qo_heads, w.num_kv_heads, w.head_dim, kv.page_size,
                             torch_dtype(w.dtype), out_dtype=out_dtype,
                             rope_theta=w.rope_theta, rope_llama31=w.rope_llama31,
                             kv_fp8=kv.dtype == "fp8_e4m3", k_scale=w.k_scale,
                             v_scale=w.v_scale, rope_interleave=w.rope_interleave)
    dec = abp.BatchDecode(params, max_batch=max(w.batch, 1), num_workers=num_workers)
    dec.plan(kv.kv_indptr, kv.kv_last_page_len)
    o, lse = dec.run(q, dev["k"], dev["v"], dev["indptr"], dev["indices"], dev["lpl"],
                     q_pos=i32(w.q_pos), kv_pos_offset=i32(w.kv_pos_offset))
    torch.cuda.synchronize()
    res = (o.float().cpu().numpy(), lse.cpu().numpy())
    if return_runner:
        return res, (dec, q, dev, o, lse)
    return res


def run_append(w, num_workers=0, out_dtype=None, dev=None):
    import torch
    kv = w.kv
    dev = dev or upload_kv(kv)
    q = wl.to_torch(w.q, w.dtype, "cuda")
    params = abp.make_params(w.num_qo_heads, w.num_kv_heads, w.head_dim, kv.page_size,
                             torch_dtype(w.dtype), out_dtype=out_dtype, causal=w.causal,
                             rope_theta=w.rope_theta, rope_llama31=w.rope_llama31,
                             rope_interleave=w.rope_interleave)
    app = abp.BatchAppend(params, max_batch=max(w.batch, 1),
                          max_qo_tokens=max(int(w.qo_indptr[-1]), 1), num_workers=num_workers)
    app.plan(w.qo_indptr, kv.kv_indptr, kv.kv_last_page_len)
    o, lse = app.run(q, dev["k"], dev["v"], i32(w.qo_indptr), dev["indptr"], dev["indices"],
                     dev["lpl"], q_pos=i32(w.q_pos), kv_pos_offset=i32(w.kv_pos_offset))
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def assert_parity(o, lse, o_ref, lse_ref, dtype, rows=None, what=""):
    """Element-wise comparison of (o, lse) with the oracle on the computed rows."""
    if rows is not None:
        o, lse, o_ref, lse_ref = o[rows], lse[rows], o_ref[rows], lse_ref[rows]
    assert np.all(np.isfinite(o)), f"{what}: non-finite o"
    inf_ref = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(lse), inf_ref), f"{what}: -inf lse pattern differs"
    do = np.max(np.abs(o - o_ref)) if o.size else 0.0
    dl = np.max(np.abs(lse[~inf_ref] - lse_ref[~inf_ref])) if (~inf_ref).any() else 0.0
    say(f"[parity] {what}: max|do| = {do:.3e} (tol {O_TOL[dtype]}), max|dlse| = {dl:.3e}")
    assert do <= O_TOL[dtype], f"{what}: max|o - o_ref| = {do}"
    assert dl <= LSE_TOL, f"{what}: max|lse - lse_ref| = {dl}"
    assert np.all(o[inf_ref] == 0), f"{what}: empty rows must be 0"


def run_bsr(w, num_workers=0, out_dtype=None, runner=None):
    """Block-sparse attention of a BsrWorkload through the C ABI."""
    import torch
    q = wl.to_torch(w.q, w.dtype, "cuda")
    k = wl.to_torch(w.k, w.dtype, "cuda")
    v = wl.to_torch(w.v, w.dtype, "cuda")
    if runner is None:
        params = abp.make_params(w.num_qo_heads, w.num_kv_heads, w.head_dim, w.C,
                                 torch_dtype(w.dtype), out_dtype=out_dtype)
        nrb = len(w.indptr) - 1
        runner = abp.BlockSparseAttention(params, max_row_blocks=max(nrb, 1),
                                          max_M=max(w.M, 1), num_workers=num_workers)
    runner.plan(w.M, w.N, w.R, w.indptr)
    o, lse = runner.run(q, k, v, i32(w.indptr), i32(w.indices))
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()
