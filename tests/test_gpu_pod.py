"""GPU checks of mixed decode + append batches (one launch whose workgroups
take the decode or the append role) against the fp64 oracle, through the C ABI.

Each part must meet the parity bar against the oracle, and must equal bit for
bit what the separate decode and append runs give with the same worker counts
(the launch runs the same worker bodies over the same sub-plans).
"""
import numpy as np
import pytest

import attention_bsr_paged_amd as abp
from attention_bsr_paged_amd import workloads as wl
from oracle import attention as ora

from gpu_helpers import assert_parity, i32, run_append, run_decode, say, torch_dtype

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    abp.load_library()


def run_pod(w, num_groups=0, decode_groups=0, out_dtype=None):
    import torch
    d, a = w.dec, w.app
    dt = d.dtype if d is not None else a.dtype
    kv0 = (d or a).kv
    k = wl.to_torch(kv0.k_pages, dt, "cuda")
    v = wl.to_torch(kv0.v_pages, dt, "cuda")
    hq, hkv = (d or a).num_qo_heads, (d or a).num_kv_heads
    params = abp.make_params(hq, hkv, 128, kv0.page_size, torch_dtype(dt), out_dtype=out_dtype,
                             causal=bool(a is not None and a.causal))
    nd = 0 if d is None else len(d.kv.kv_indptr) - 1
    na = 0 if a is None else len(a.kv.kv_indptr) - 1
    nq = 0 if a is None else int(a.qo_indptr[-1])
    pod = abp.PodAttention(params, max(nd, 1), max(na, 1), max(nq, 1), num_groups=num_groups)
    plan = pod.plan(None if d is None else d.kv.kv_indptr,
                    None if d is None else d.kv.kv_last_page_len,
                    None if a is None else a.qo_indptr, None if a is None else a.kv.kv_indptr,
                    None if a is None else a.kv.kv_last_page_len, decode_groups=decode_groups)
    say(f"[pod] groups {plan.num_groups}: decode {plan.decode.num_workers}, "
        f"append {plan.append.num_workers}")
    qd = None if d is None else wl.to_torch(d.q, dt, "cuda")
    qa = None if a is None else wl.to_torch(a.q, dt, "cuda")
    (od, ld), (oa, la) = pod.run(
        qd, qa, k, v, None if d is None else i32(d.kv.kv_indptr),
        None if d is None else i32(d.kv.kv_indices),
        None if d is None else i32(d.kv.kv_last_page_len), None if a is None else i32(a.qo_indptr),
        None if a is None else i32(a.kv.kv_indptr), None if a is None else i32(a.kv.kv_indices),
        None if a is None else i32(a.kv.kv_last_page_len))
    torch.cuda.synchronize()
    dres = None if d is None else (od.float().cpu().numpy(), ld.cpu().numpy())
    ares = None if a is None else (oa.float().cpu().numpy(), la.cpu().numpy())
    return dres, ares, plan


def small_mixed(seed, G, causal, dtype="bf16", hkv=4):
    dec = wl.small_decode(seed, [0, 1, 15, 16, 17, 300, 1000, 64, 2049], 16, hkv * G, hkv,
                          dtype=dtype)
    app = wl.small_append(seed + 1, [1, 37, 128, 200, 64], [5, 100, 300, 700, 64], 16, hkv * G,
                          hkv, dtype=dtype, causal=causal)
    return wl.mixed_batch(dec, app, f"small_mixed_s{seed}")


@pytest.mark.parametrize("G", [4, 8])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("groups,decode_groups", [(0, 0), (16, 0), (5, 2), (2, 1)])
def test_pod_parity_and_same_as_separate_runs(G, causal, groups, decode_groups):
    dtype = "fp16" if G == 8 else "bf16"
    w = small_mixed(700 + G + causal, G, causal, dtype)
    say(f"[case] pod G={G} causal={causal} groups={groups} decode_groups={decode_groups}")
    (od, ld), (oa, la), plan = run_pod(w, groups, decode_groups)
    od_ref, ld_ref = ora.decode_workload(w.dec)
    oa_ref, la_ref = ora.append_workload(w.app)
    assert_parity(od, ld, od_ref, ld_ref, dtype, what="pod decode part")
    assert_parity(oa, la, oa_ref, la_ref, dtype, what="pod append part")
    od2, ld2 = run_decode(w.dec, num_workers=plan.decode.num_workers)
    oa2, la2 = run_append(w.app, num_workers=plan.append.num_workers)
    assert np.array_equal(od, od2) and np.array_equal(ld, ld2), "decode part differs"
    assert np.array_equal(oa, oa2) and np.array_equal(la, la2), "append part differs"


def test_pod_one_part_only():
    w = small_mixed(720, 4, True)
    only_app = wl.PodWorkload("append only", None, w.app)
    _, (oa, la), plan = run_pod(only_app)
    assert plan.decode.num_workers == 0
    oa_ref, la_ref = ora.append_workload(w.app)
    assert_parity(oa, la, oa_ref, la_ref, "bf16", what="pod append only")
    only_dec = wl.PodWorkload("decode only", w.dec, None)
    (od, ld), _, plan = run_pod(only_dec)
    assert plan.append.num_workers == 0
    od_ref, ld_ref = ora.decode_workload(w.dec)
    assert_parity(od, ld, od_ref, ld_ref, "bf16", what="pod decode only")


def test_pod_f32_out():
    import torch
    w = small_mixed(730, 4, True)
    (od, ld), (oa, la), _ = run_pod(w, 16, 0, out_dtype=torch.float32)
    od_ref, ld_ref = ora.decode_workload(w.dec)
    oa_ref, la_ref = ora.append_workload(w.app)
    assert_parity(od, ld, od_ref, ld_ref, "bf16", what="pod decode f32 out")
    assert_parity(oa, la, oa_ref, la_ref, "bf16", what="pod append f32 out")


def test_pod_benchmark_batch_sampled():
    """The benchmark's mixed batch in its launch configuration (default split),
    checked on sampled decode requests and sampled query tokens."""
    w = wl.pod_mixed()
    (od, ld), (oa, la), plan = run_pod(w)
    assert plan.decode.num_workers > 0 and plan.append.num_workers > 0
    rng = np.random.default_rng(5)
    nd = len(w.dec.kv.kv_indptr) - 1
    bids = sorted(set([0, nd - 1] + list(rng.choice(nd, 6, replace=False))))
    od_ref, ld_ref = ora.decode_workload(w.dec, batch_ids=bids)
    assert_parity(od, ld, od_ref, ld_ref, "bf16", rows=bids, what="pod bench decode sample")
    toks = []
    for b in range(len(w.app.qo_indptr) - 1):
        q0, q1 = int(w.app.qo_indptr[b]), int(w.app.qo_indptr[b + 1])
        toks += [q0, q1 - 1] + list(rng.integers(q0, q1, size=4))
    toks = sorted(set(toks))
    oa_ref, la_ref = ora.append_workload(w.app, token_ids=toks)
    assert_parity(oa, la, oa_ref, la_ref, "bf16", rows=toks, what="pod bench append sample")
    assert np.all(np.isfinite(od)) and np.all(np.isfinite(oa))


def test_pod_graph_replay_with_fixed_split():
    """run() captured in a hipGraph: every replay equals the eager result, also
    after a re-plan that keeps the split (decode_groups) and the capacities."""
    import torch
    w = small_mixed(740, 4, True)
    d, a = w.dec, w.app
    k = wl.to_torch(d.kv.k_pages, "bf16", "cuda")
    v = wl.to_torch(d.kv.v_pages, "bf16", "cuda")
    params = abp.make_params(16, 4, 128, 16, torch.bfloat16, causal=True)
    nd, na, nq = len(d.kv.kv_indptr) - 1, len(a.kv.kv_indptr) - 1, int(a.qo_indptr[-1])
    pod = abp.PodAttention(params, nd, na, nq, num_groups=32)
    qd, qa = wl.to_torch(d.q, "bf16", "cuda"), wl.to_torch(a.q, "bf16", "cuda")
    D = [i32(d.kv.kv_indptr), i32(d.kv.kv_indices), i32(d.kv.kv_last_page_len)]
    A = [i32(a.qo_indptr), i32(a.kv.kv_indptr), i32(a.kv.kv_indices), i32(a.kv.kv_last_page_len)]
    od, oa = torch.empty_like(qd), torch.empty_like(qa)
    ld = torch.empty(qd.shape[:2], dtype=torch.float32, device="cuda")
    la = torch.empty(qa.shape[:2], dtype=torch.float32, device="cuda")

    def run(stream=None):
        pod.run(qd, qa, k, v, *D, *A, o_decode=od, lse_decode=ld, o_append=oa, lse_append=la,
                stream=stream)

    def outs():
        return [t.clone() for t in (od, ld, oa, la)]

    pod.plan(d.kv.kv_indptr, d.kv.kv_last_page_len, a.qo_indptr, a.kv.kv_indptr,
             a.kv.kv_last_page_len, decode_groups=12)
    run()
    torch.cuda.synchronize()
    eager1 = outs()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            run(s)
    torch.cuda.synchronize()
    for _ in range(3):
        for t in (od, oa):
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(x, y) for x, y in zip(outs(), eager1))
    # re-plan with shorter last pages of the decode requests (same page table
    # arrays, same capacities, same split)
    lpl2 = np.where(np.diff(d.kv.kv_indptr) > 0, np.maximum(1, d.kv.kv_last_page_len // 2),
                    d.kv.kv_last_page_len).astype(np.int32)
    D[2].copy_(i32(lpl2))
    plan = pod.plan(d.kv.kv_indptr, lpl2, a.qo_indptr, a.kv.kv_indptr, a.kv.kv_last_page_len,
                    decode_groups=12)
    assert plan.decode.num_workers == 12
    run()
    torch.cuda.synchronize()
    eager2 = outs()
    assert not torch.equal(eager2[0], eager1[0])
    for _ in range(3):
        for t in (od, oa):
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert all(torch.equal(x, y) for x, y in zip(outs(), eager2))
    d.kv.kv_last_page_len = lpl2
    od_ref, ld_ref = ora.decode_workload(d)
    assert_parity(eager2[0].float().cpu().numpy(), eager2[1].cpu().numpy(), od_ref, ld_ref,
                  "bf16", what="pod decode after re-plan")
