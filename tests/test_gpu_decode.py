"""GPU parity of the paged decode path (C ABI through the binding) against the
fp64 oracle, plus the invariants the method implies, determinism, a poisoned
workspace and graph replay."""
import numpy as np
import pytest

import attention_bsr_paged_amd as abp
from attention_bsr_paged_amd import workloads as wl
from oracle import attention as ora

from gpu_helpers import assert_parity, i32, run_decode, say, upload_kv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    abp.load_library()


LENGTHS = [0, 1, 15, 16, 17, 63, 64, 65, 200, 1000, 2500]


@pytest.mark.parametrize("P", [1, 3, 16, 256])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_small_decode_parity(P, G):
    say(f"[case] small decode P={P} G={G}")
    hkv = 2
    w = wl.small_decode(100 + P * 10 + G, LENGTHS, P, hkv * G, hkv, dtype="bf16")
    o_ref, l_ref = ora.decode_workload(w)
    for W in (1, 7, 64):
        o, l = run_decode(w, num_workers=W)
        assert_parity(o, l, o_ref, l_ref, "bf16", what=f"P{P} G{G} W{W}")


@pytest.mark.parametrize("hkv", [4, 8, 12, 16])
@pytest.mark.parametrize("G", [1, 4])
@pytest.mark.parametrize("rope", [False, True])
def test_head_group_tiles(hkv, G, rope):
    """kv head counts that are multiples of 4, where a decode tile holds 4
    consecutive heads and every wave of a workgroup owns one of them (1, 2, 3
    or 4 tiles per request). Page sizes 3 (per-token path) and 16, grids of 1,
    7 and 64 workers, with and without RoPE."""
    for P in (3, 16):
        say(f"[case] head groups hkv={hkv} G={G} rope={rope} P={P}")
        w = wl.small_decode(400 + 10 * hkv + G + P, [0, 1, 17, 64, 65, 700, 1500], P, hkv * G,
                            hkv, dtype="bf16")
        if rope:
            w.rope_theta = 500000.0
            w.kv_pos_offset = np.array([0, 5, 100, 7000, 3, 0, 64], np.int32)
            w.q_pos = (w.kv_pos_offset + w.kv.kv_len - 1).astype(np.int32)
        o_ref, l_ref = ora.decode_workload(w)
        for W in (1, 7, 64):
            o, l = run_decode(w, num_workers=W)
            assert_parity(o, l, o_ref, l_ref, "bf16", what=f"hkv{hkv} G{G} rope{rope} P{P} W{W}")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("out", [None, "fp32"])
def test_dtypes(dtype, out):
    say(f"[case] dtype {dtype} out {out}")
    w = wl.small_decode(7, [5, 77, 300, 1], 16, 8, 2, dtype=dtype)
    o_ref, l_ref = ora.decode_workload(w)
    import torch
    o, l = run_decode(w, num_workers=9, out_dtype=None if out is None else torch.float32)
    assert_parity(o, l, o_ref, l_ref, dtype, what=f"{dtype}->{out}")


def test_single_decode_mha_fp16():
    """Single request, 32 qo = 32 kv heads, kv_len 2048 in 128 shuffled pages of 16, fp16."""
    w = wl.single_decode_mha()
    o_ref, l_ref = ora.decode_workload(w)
    for W in (0, 1, 32):
        o, l = run_decode(w, num_workers=W)
        assert_parity(o, l, o_ref, l_ref, "fp16", what=f"single decode W{W}")


def test_single_decode_contiguous_api():
    """The pages' example call: q [32,128], k/v [2048,32,128] fp16 -> o [32,128]."""
    import torch
    w = wl.single_decode_mha()
    kv = w.kv
    # logical (contiguous) K/V of the request
    K = ora.walk_pages(kv.k_pages, kv.kv_indptr, kv.kv_indices, kv.kv_last_page_len, 16, 0)
    V = ora.walk_pages(kv.v_pages, kv.kv_indptr, kv.kv_indices, kv.kv_last_page_len, 16, 0)
    q = wl.to_torch(w.q[0], "fp16", "cuda")
    o, lse = abp.single_decode_with_kv_cache(q, wl.to_torch(K, "fp16", "cuda"),
                                             wl.to_torch(V, "fp16", "cuda"), return_lse=True)
    assert tuple(o.shape) == (32, 128)
    o_ref, l_ref = ora.decode_workload(w)
    assert_parity(o.float().cpu().numpy()[None], lse.cpu().numpy()[None], o_ref, l_ref, "fp16",
                  what="single_decode_with_kv_cache")


@pytest.mark.parametrize("name", ["batch_decode", "skewed_decode"])
def test_named_decode_workloads(name):
    """Full-size batch and skewed decode in the launch configuration the benchmark
    times (default workers), every request compared."""
    w = wl.WORKLOADS[name]()
    say(f"[case] {w.name}")
    o, l = run_decode(w)
    o_ref, l_ref = ora.decode_workload(w)
    assert_parity(o, l, o_ref, l_ref, w.dtype, what=f"{name}, all requests")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))


def test_worker_count_invariance_and_determinism():
    w = wl.small_decode(11, [3000, 17, 900, 4096, 1], 16, 32, 8)
    o_ref, l_ref = ora.decode_workload(w)
    outs = []
    for W in (1, 13, 256, 512, 2048):
        o, l = run_decode(w, num_workers=W)
        assert_parity(o, l, o_ref, l_ref, "bf16", what=f"W{W}")
        outs.append((o, l))
    o2, l2 = run_decode(w, num_workers=2048)
    assert np.array_equal(outs[-1][0], o2) and np.array_equal(outs[-1][1], l2)


def test_page_permutation_invariance():
    w = wl.small_decode(12, [700, 33, 1200], 16, 8, 2, extra_pages=9)
    o1, l1 = run_decode(w, num_workers=16)
    kv = w.kv
    perm = np.random.Generator(np.random.PCG64(3)).permutation(kv.num_pages)
    kp = np.empty_like(kv.k_pages)
    vp = np.empty_like(kv.v_pages)
    kp[perm] = kv.k_pages
    vp[perm] = kv.v_pages
    kv.k_pages, kv.v_pages = kp, vp
    kv.kv_indices = perm[kv.kv_indices].astype(np.int32)
    o2, l2 = run_decode(w, num_workers=16)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_poisoned_workspace():
    """NaN in the device workspace's partial region must never reach the output."""
    import torch
    w = wl.small_decode(13, [2000, 3000, 50], 16, 8, 2)
    kv = w.kv
    dev = upload_kv(kv)
    params = abp.make_params(8, 2, 128, 16, torch.bfloat16)
    dec = abp.BatchDecode(params, max_batch=3, num_workers=64)
    plan = dec.plan(kv.kv_indptr, kv.kv_last_page_len)
    assert plan.num_merges > 0
    torch.cuda.synchronize()
    part = dec.dev_ws[plan.partial_offset:]
    part.view(torch.float32)[: part.numel() // 4].fill_(float("nan"))
    q = wl.to_torch(w.q, "bf16", "cuda")
    o, l = dec.run(q, dev["k"], dev["v"], dev["indptr"], dev["indices"], dev["lpl"])
    torch.cuda.synchronize()
    o_ref, l_ref = ora.decode_workload(w)
    assert_parity(o.float().cpu().numpy(), l.cpu().numpy(), o_ref, l_ref, "bf16", what="poisoned")


def test_graph_replay_after_replan():
    """run() captured once in a hipGraph stays valid after a re-plan with the same
    capacities; every replay equals the eager result."""
    import torch
    w1 = wl.small_decode(14, [1000, 2000, 300, 64], 16, 8, 2, extra_pages=200)
    kv = w1.kv
    dev = upload_kv(kv)
    params = abp.make_params(8, 2, 128, 16, torch.bfloat16)
    dec = abp.BatchDecode(params, max_batch=4, num_workers=32)
    q = wl.to_torch(w1.q, "bf16", "cuda")
    o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    dec.plan(kv.kv_indptr, kv.kv_last_page_len)
    dec.run(q, dev["k"], dev["v"], dev["indptr"], dev["indices"], dev["lpl"], o=o, lse=lse)
    torch.cuda.synchronize()
    eager1 = (o.clone(), lse.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            dec.run(q, dev["k"], dev["v"], dev["indptr"], dev["indices"], dev["lpl"], o=o,
                    lse=lse, stream=s)
    torch.cuda.synchronize()
    for _ in range(3):
        o.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eager1[0]) and torch.equal(lse, eager1[1])
    # re-plan: shorter lengths over the same page table arrays (same capacities)
    lens = np.array([500, 17, 300, 0])
    indptr, _, lpl = wl.page_table(lens, 16, np.arange(10 ** 6))
    indices = kv.kv_indices[: indptr[-1]].copy()   # first pages of the pool order
    dev["indptr"].copy_(i32(indptr).to(torch.int32))
    dev["lpl"].copy_(i32(lpl))
    dev["indices"][: len(indices)].copy_(i32(indices))
    dec.plan(indptr, lpl)
    torch.cuda.synchronize()
    dec.run(q, dev["k"], dev["v"], dev["indptr"], dev["indices"], dev["lpl"], o=o, lse=lse)
    torch.cuda.synchronize()
    eager2 = (o.clone(), lse.clone())
    for _ in range(3):
        o.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eager2[0]) and torch.equal(lse, eager2[1])
    kv2 = wl.PagedKV(16, 2, 128, "bf16", lens, indptr, indices, lpl, kv.k_pages, kv.v_pages)
    o_ref, l_ref = ora.paged_decode(w1.q, kv2.k_pages, kv2.v_pages, indptr, indices, lpl, 16,
                                    "bf16", 2)
    assert_parity(eager2[0].float().cpu().numpy(), eager2[1].cpu().numpy(), o_ref, l_ref, "bf16",
                  what="replanned")


def test_plan_upload_paths_and_replan_sequence():
    """The plan reaches the device workspace either through a kernel that reads
    the pinned host workspace (the binding's) or through hipMemcpyAsync (a
    pageable host workspace). Both give the same bits, and a sequence of
    different plans through one workspace each gives the oracle's result."""
    import ctypes
    import torch
    lib = abp.load_library()
    params = abp.make_params(8, 2, 128, 16, torch.bfloat16)
    dec = abp.BatchDecode(params, max_batch=3, num_workers=24)
    stream = torch.cuda.current_stream().cuda_stream
    for i, lens in enumerate(([700, 5, 64], [17, 2000, 0], [300, 301, 302], [1, 1, 1])):
        w = wl.small_decode(31 + i, lens, 16, 8, 2)
        say(f"[case] upload paths, lengths {lens}")
        kv = w.kv
        dev = upload_kv(kv)
        q = wl.to_torch(w.q, "bf16", "cuda")
        plan = dec.plan(kv.kv_indptr, kv.kv_last_page_len)
        assert plan.upload_path == 1, "pinned host workspace should be read by the upload kernel"
        o, l = dec.run(q, dev["k"], dev["v"], dev["indptr"], dev["indices"], dev["lpl"])
        torch.cuda.synchronize()
        o_ref, l_ref = ora.decode_workload(w)
        assert_parity(o.float().cpu().numpy(), l.cpu().numpy(), o_ref, l_ref, "bf16",
                      what=f"pinned upload {lens}")
        host = np.zeros(dec.host_ws.numel(), np.uint8)   # pageable
        indptr = np.ascontiguousarray(kv.kv_indptr, np.int32)
        lpl = np.ascontiguousarray(kv.kv_last_page_len, np.int32)
        p2 = abp.AbpPlan()
        st = lib.abp_decode_plan(ctypes.byref(params), 3, indptr.ctypes.data, lpl.ctypes.data, 3,
                                 24, host.ctypes.data, host.nbytes, dec.dev_ws.data_ptr(),
                                 dec.dev_ws.numel(), stream, ctypes.byref(p2))
        assert st == 0, abp.abp_last_error()
        torch.cuda.synchronize()
        assert p2.upload_path == 0
        assert p2.fingerprint == plan.fingerprint and p2.num_segments == plan.num_segments
        dec.plan_struct = p2
        o2, l2 = dec.run(q, dev["k"], dev["v"], dev["indptr"], dev["indices"], dev["lpl"])
        torch.cuda.synchronize()
        assert torch.equal(o2, o) and torch.equal(l2, l)


@pytest.mark.parametrize("in_dt,out_dt", [("fp32", "bf16"), ("bf16", "bf16"), ("fp16", "fp32")])
def test_merge_state_kernel(in_dt, out_dt):
    import torch
    tdt = {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}
    rng = np.random.Generator(np.random.PCG64(21))
    rows = 1000
    oa = rng.standard_normal((rows, 128)).astype(np.float32)
    ob = rng.standard_normal((rows, 128)).astype(np.float32)
    la = (rng.standard_normal(rows) * 3).astype(np.float32)
    lb = (rng.standard_normal(rows) * 3).astype(np.float32)
    la[:5] = -np.inf
    lb[3:8] = -np.inf
    ta = torch.from_numpy(oa).to("cuda", tdt[in_dt])
    tb = torch.from_numpy(ob).to("cuda", tdt[in_dt])
    o, l = abp.merge_state(ta, torch.from_numpy(la).cuda(), tb, torch.from_numpy(lb).cuda(),
                           out_dtype=tdt[out_dt])
    torch.cuda.synchronize()
    o_ref, l_ref = ora.merge([(ta.double().cpu().numpy(), la), (tb.double().cpu().numpy(), lb)])
    tol = {"fp32": 1e-5, "bf16": 2e-2, "fp16": 1e-2}[out_dt]
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isneginf(l.cpu().numpy()), ~fin)
    assert np.max(np.abs(o.double().cpu().numpy() - o_ref)) <= tol + 1e-6
    assert np.max(np.abs(l.cpu().numpy()[fin] - l_ref[fin])) <= 1e-5


def test_merge_states_kernel():
    import torch
    rng = np.random.Generator(np.random.PCG64(22))
    n, rows = 5, 333
    o = rng.standard_normal((n, rows, 128)).astype(np.float32)
    l = (rng.standard_normal((n, rows)) * 2).astype(np.float32)
    l[:, :3] = -np.inf
    l[2, 10] = -np.inf
    om, lm = abp.merge_states(torch.from_numpy(o).cuda(), torch.from_numpy(l).cuda())
    torch.cuda.synchronize()
    o_ref, l_ref = ora.merge([(o[i].astype(np.float64), l[i]) for i in range(n)])
    fin = np.isfinite(l_ref)
    assert np.max(np.abs(om.double().cpu().numpy() - o_ref)) <= 1e-5
    assert np.max(np.abs(lm.cpu().numpy()[fin] - l_ref[fin])) <= 1e-5
    assert np.all(np.isneginf(lm.cpu().numpy()[~fin]))


def test_empty_batches():
    """batch 0 plans and runs (no work, nothing written); a batch whose requests
    all have no pages gives (0, -inf) for every row."""
    import torch
    params = abp.make_params(8, 2, 128, 16, torch.bfloat16)
    dec = abp.BatchDecode(params, max_batch=4, num_workers=8)
    plan = dec.plan(np.zeros(1, np.int32), np.zeros(0, np.int32))
    assert plan.num_tiles == 0
    dev = torch.zeros(1, dtype=torch.int32, device="cuda")
    kp = torch.zeros((1, 16, 2, 128), dtype=torch.bfloat16, device="cuda")
    q0 = torch.zeros((0, 8, 128), dtype=torch.bfloat16, device="cuda")
    o, l = dec.run(q0, kp, kp, dev, dev, dev)
    torch.cuda.synchronize()
    assert o.shape == (0, 8, 128)
    # three requests without pages
    plan = dec.plan(np.zeros(4, np.int32), np.zeros(3, np.int32))
    q = torch.randn((3, 8, 128), device="cuda").to(torch.bfloat16)
    o, l = dec.run(q, kp, kp, torch.zeros(4, dtype=torch.int32, device="cuda"), dev,
                   torch.zeros(3, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))
    # append with no query tokens at all
    pa = abp.make_params(8, 2, 128, 16, torch.bfloat16, causal=True)
    app = abp.BatchAppend(pa, max_batch=2, max_qo_tokens=8, num_workers=8)
    plan = app.plan(np.zeros(3, np.int32), np.array([0, 1, 2], np.int32), np.array([5, 9], np.int32))
    assert plan.num_tiles == 0
    qa = torch.zeros((0, 8, 128), dtype=torch.bfloat16, device="cuda")
    o, l = app.run(qa, kp, kp, torch.zeros(3, dtype=torch.int32, device="cuda"),
                   torch.tensor([0, 1, 2], dtype=torch.int32, device="cuda"),
                   torch.zeros(2, dtype=torch.int32, device="cuda"),
                   torch.tensor([5, 9], dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert o.shape == (0, 8, 128)


@pytest.mark.parametrize("P,G,hkv,dtype", [(16, 4, 4, "bf16"), (32, 8, 4, "fp16"),
                                           (64, 4, 8, "bf16"), (16, 8, 12, "bf16")])
def test_matrix_core_decode_chunk_edges(P, G, hkv, dtype):
    """The matrix-core decode path (power-of-two pages >= 16, kv heads a multiple
    of 4, G 4 or 8): lengths around its 16-token tiles and 32-token chunks, odd
    and even chunk counts per segment, and segments cut at every worker count."""
    lens = [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 97, 128, 1000]
    w = wl.small_decode(900 + P + G + hkv, lens, P, G * hkv, hkv, dtype=dtype)
    o_ref, l_ref = ora.decode_workload(w)
    for W in (1, 7, 64, 0):
        o, l = run_decode(w, num_workers=W)
        assert_parity(o, l, o_ref, l_ref, dtype, what=f"mfma decode P{P} G{G} hkv{hkv} W{W}")


def test_one_worker_per_tile_plan():
    """The plan without load balancing (ABP_WORKERS_PER_TILE: one worker per
    tile, no split, no partial states) gives the same attention."""
    w = wl.small_decode(13, [0, 1, 17, 700, 3000, 64], 16, 32, 8)
    o_ref, l_ref = ora.decode_workload(w)
    o, l = run_decode(w, num_workers=abp.ABP_WORKERS_PER_TILE)
    assert_parity(o, l, o_ref, l_ref, "bf16", what="one worker per tile")
    w3 = wl.small_decode(14, [0, 5, 300, 2000], 3, 8, 2)
    o_ref, l_ref = ora.decode_workload(w3)
    o, l = run_decode(w3, num_workers=abp.ABP_WORKERS_PER_TILE)
    assert_parity(o, l, o_ref, l_ref, "bf16", what="one worker per tile, P 3")


@pytest.mark.parametrize("variant", ["rotate_half", "interleaved", "llama31"])
@pytest.mark.parametrize("G,P,dtype", [(4, 16, "bf16"), (8, 16, "fp16"), (4, 256, "fp16"),
                                       (8, 64, "bf16")])
def test_rope_decode_matrix_cores(variant, G, P, dtype):
    """RoPE decode on the matrix-core path (kv heads a multiple of 4, G 4 or 8,
    power-of-two pages >= 16): q and K rotated in fp32, hi/lo products. Key
    offsets and query positions vary per request; slots without a token hold
    NaN / inf."""
    say(f"[case] matrix-core rope decode {variant} G={G} P={P} {dtype}")
    lens = [0, 1, 15, 16, 17, 33, 64, 65, 500, 1000, 2100]
    w = wl.small_decode(600 + G + P, lens, P, 8 * G, 8, dtype=dtype)
    w.kv = wl.poison_unwritten(w.kv)
    w.rope_theta = 500000.0
    w.rope_interleave = variant == "interleaved"
    w.rope_llama31 = abp.LLAMA31_ROPE if variant == "llama31" else None
    w.kv_pos_offset = (np.arange(len(lens)) * 37 % 5000).astype(np.int32)
    w.q_pos = (w.kv_pos_offset + w.kv.kv_len - 1 + np.arange(len(lens)) % 3).astype(np.int32)
    o_ref, l_ref = ora.decode_workload(w)
    for W in (1, 13, 0):
        o, l = run_decode(w, num_workers=W)
        assert_parity(o, l, o_ref, l_ref, dtype, what=f"mfma rope {variant} G{G} P{P} W{W}")
