"""GPU parity of the append / prefill (MFMA) path, fused RoPE and the cascade
(composable formats) path against the fp64 oracle."""
import numpy as np
import pytest

import attention_bsr_paged_amd as abp
from attention_bsr_paged_amd import workloads as wl
from oracle import attention as ora

from gpu_helpers import assert_parity, i32, run_append, run_decode, say, upload_kv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    abp.load_library()


QO = [1, 5, 31, 32, 33, 64, 130, 300]
KV_EXTRA = [0, 3, 64, 1, 200, 17, 1000, 65]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("P", [1, 3, 16, 256])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_small_append_parity(causal, P, G):
    say(f"[case] small append causal={causal} P={P} G={G}")
    kv = [q + e for q, e in zip(QO, KV_EXTRA)]
    w = wl.small_append(200 + P + G, QO, kv, P, 2 * G, 2, dtype="bf16", causal=causal)
    o_ref, l_ref = ora.append_workload(w)
    for W in (1, 9, 0):
        o, l = run_append(w, num_workers=W)
        assert_parity(o, l, o_ref, l_ref, "bf16", what=f"append c{int(causal)} P{P} G{G} W{W}")


@pytest.mark.parametrize("G", [2, 16])
def test_group_sizes_fp16(G):
    w = wl.small_append(300 + G, [7, 70, 129], [9, 500, 129], 16, 2 * G, 2, dtype="fp16",
                        causal=True)
    o_ref, l_ref = ora.append_workload(w)
    o, l = run_append(w, num_workers=13)
    assert_parity(o, l, o_ref, l_ref, "fp16", what=f"append fp16 G{G}")


def test_empty_and_zero_query_requests():
    """Requests with no queries write nothing; a non-causal request with no keys gives (0, -inf)."""
    w = wl.small_append(310, [0, 4, 0, 3], [10, 0, 5, 7], 16, 8, 2, causal=False)
    o_ref, l_ref = ora.append_workload(w)
    o, l = run_append(w, num_workers=5)
    assert_parity(o, l, o_ref, l_ref, "bf16", what="empty requests")


def test_ragged_append_sampled():
    """Full ragged causal append (16 requests, qo U{128..1024} onto kv U{1024..8192},
    GQA 32/8, bf16) in the launch configuration the benchmark times, compared on
    at least 64 query tokens of every request: the first and last, both sides
    of every 64-token query-tile boundary, and random ones."""
    w = wl.ragged_append_causal()
    say(f"[case] {w.name}")
    o, l = run_append(w)
    rng = np.random.Generator(np.random.PCG64(9))
    toks = []
    for b in range(w.batch):
        q0, q1 = int(w.qo_indptr[b]), int(w.qo_indptr[b + 1])
        mine = {q0, q1 - 1}
        mine |= {t for j in range(q0 + 64, q1, 64) for t in (j - 1, j)}
        mine |= set(int(t) for t in rng.choice(np.arange(q0, q1), size=64, replace=False))
        assert len(mine) >= 64
        toks += sorted(mine)
    toks = sorted(set(toks))
    o_ref, l_ref = ora.append_workload(w, token_ids=toks)
    assert_parity(o, l, o_ref, l_ref, "bf16", rows=toks, what="ragged append sampled")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))


def test_append_worker_invariance_and_determinism():
    w = wl.small_append(320, [100, 257], [900, 2000], 16, 32, 8, causal=True)
    o_ref, l_ref = ora.append_workload(w)
    prev = None
    for W in (1, 3, 64, 256):
        o, l = run_append(w, num_workers=W)
        assert_parity(o, l, o_ref, l_ref, "bf16", what=f"W{W}")
    o1, l1 = run_append(w, num_workers=64)
    o2, l2 = run_append(w, num_workers=64)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("W", [16, 32, 64, 224])
@pytest.mark.parametrize("rope", [False, True])
def test_co_scheduled_plans(W, rope):
    """Worker counts whose plans run K = 2, 4, 8, 4 consecutive query tiles of
    one (request, kv head) side by side: ragged query tails, causal requests of
    different lengths (idle lanes, units mixing kv heads), with and without
    RoPE."""
    say(f"[case] co-scheduled append W={W} rope={rope}")
    w = wl.small_append(330 + W, [300, 7, 129, 64, 33], [2100, 70, 900, 64, 1000], 16, 8, 2,
                        causal=True)
    if rope:
        w.rope_theta = 500000.0
    o_ref, l_ref = ora.append_workload(w)
    o, l = run_append(w, num_workers=W)
    assert_parity(o, l, o_ref, l_ref, "bf16", what=f"co-scheduled W{W} rope{int(rope)}")


def test_merge_modes_and_graph_replay_across_them():
    """A tile split into more than 4 partials is merged by the merge kernel, at
    most 4 inside the append kernel. Both give the oracle's result, and a run
    captured in a graph under one mode replays correctly after a re-plan that
    selects the other (the launch sequence does not depend on the plan)."""
    import torch
    w = wl.small_append(325, [40, 7], [3000, 50], 16, 8, 2, causal=True, extra_pages=64)
    kv = w.kv
    dev = upload_kv(kv)
    q = wl.to_torch(w.q, "bf16", "cuda")
    params = abp.make_params(8, 2, 128, 16, torch.bfloat16, causal=True)
    app = abp.BatchAppend(params, max_batch=2, max_qo_tokens=64, num_workers=64)
    plan = app.plan(w.qo_indptr, kv.kv_indptr, kv.kv_last_page_len)
    torch.cuda.synchronize()
    arr = abp.decode_plan_arrays(app.host_ws.numpy(), plan)
    assert int(arr["merge_kernel"][0]) == 1 and int(arr["tile_num_partials"].max()) > 4
    o = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device="cuda")
    qo = i32(w.qo_indptr)
    app.run(q, dev["k"], dev["v"], qo, dev["indptr"], dev["indices"], dev["lpl"], o=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = ora.append_workload(w)
    assert_parity(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "bf16",
                  what="merge kernel mode")
    eager1 = (o.clone(), lse.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            app.run(q, dev["k"], dev["v"], qo, dev["indptr"], dev["indices"], dev["lpl"], o=o,
                    lse=lse, stream=s)
    torch.cuda.synchronize()
    for _ in range(2):
        o.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eager1[0]) and torch.equal(lse, eager1[1])
    # re-plan with short keys: every tile fits in a few blocks, merged in place
    lens = np.array([64, 20])
    indptr, _, lpl = wl.page_table(lens, 16, np.arange(10 ** 6))
    indices = kv.kv_indices[: indptr[-1]].copy()
    dev["indptr"].copy_(i32(indptr))
    dev["lpl"].copy_(i32(lpl))
    dev["indices"][: len(indices)].copy_(i32(indices))
    qo_b = np.array([0, 40, 47], np.int32)
    plan = app.plan(qo_b, indptr, lpl)
    torch.cuda.synchronize()
    arr = abp.decode_plan_arrays(app.host_ws.numpy(), plan)
    assert int(arr["merge_kernel"][0]) == 0
    qo.copy_(i32(qo_b))
    app.run(q, dev["k"], dev["v"], qo, dev["indptr"], dev["indices"], dev["lpl"], o=o, lse=lse)
    torch.cuda.synchronize()
    eager2 = (o.clone(), lse.clone())
    for _ in range(2):
        o.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, eager2[0]) and torch.equal(lse, eager2[1])
    kv2 = wl.PagedKV(16, 2, 128, "bf16", lens, indptr, indices, lpl, kv.k_pages, kv.v_pages)
    o_ref2, l_ref2 = ora.paged_append(w.q, qo_b, kv2.k_pages, kv2.v_pages, indptr, indices, lpl,
                                      16, "bf16", 2, causal=True)
    assert_parity(eager2[0].float().cpu().numpy(), eager2[1].cpu().numpy(), o_ref2, l_ref2,
                  "bf16", what="merged in place after re-plan")


# ----------------------------------------------------------------------------
# fused RoPE
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("P", [3, 16])
def test_rope_decode_parity(P):
    w = wl.small_decode(330 + P, [1, 40, 700, 3000], P, 8, 2)
    w.rope_theta = 500000.0
    rng = np.random.Generator(np.random.PCG64(331))
    w.kv_pos_offset = rng.integers(0, 9000, size=w.batch).astype(np.int32)
    w.q_pos = (w.kv_pos_offset + w.kv.kv_len + rng.integers(-5, 5, size=w.batch)).astype(np.int32)
    o_ref, l_ref = ora.decode_workload(w)
    o, l = run_decode(w, num_workers=11)
    assert_parity(o, l, o_ref, l_ref, "bf16", what=f"rope decode P{P}")
    # defaults: q at kv_len - 1, keys from 0
    w.q_pos = None
    w.kv_pos_offset = None
    o_ref, l_ref = ora.decode_workload(w)
    o, l = run_decode(w, num_workers=11)
    assert_parity(o, l, o_ref, l_ref, "bf16", what=f"rope decode defaults P{P}")


@pytest.mark.parametrize("causal", [True, False])
def test_rope_append_parity(causal):
    w = wl.small_append(340, [3, 90, 200], [50, 400, 900], 16, 8, 2, causal=causal)
    w.rope_theta = 500000.0
    o_ref, l_ref = ora.append_workload(w)
    o, l = run_append(w, num_workers=7)
    assert_parity(o, l, o_ref, l_ref, "bf16", what=f"rope append c{int(causal)}")


@pytest.mark.parametrize("dtype,G", [("fp16", 8), ("bf16", 1)])
def test_rope_decode_dtype_and_group(dtype, G):
    """RoPE decode in fp16 and at the largest and smallest groups (G = 8 is the
    variant with the most registers)."""
    w = wl.small_decode(360 + G, [2, 63, 500, 1300], 16, 2 * G, 2, dtype=dtype)
    w.rope_theta = 500000.0
    w.kv_pos_offset = np.array([0, 100, 7000, 3], np.int32)
    w.q_pos = (w.kv_pos_offset + w.kv.kv_len - 1).astype(np.int32)
    o_ref, l_ref = ora.decode_workload(w)
    o, l = run_decode(w, num_workers=17)
    assert_parity(o, l, o_ref, l_ref, dtype, what=f"rope decode {dtype} G{G}")


@pytest.mark.parametrize("G,dtype,causal", [(1, "bf16", True), (2, "fp16", False),
                                            (8, "fp16", True), (16, "bf16", True)])
def test_rope_append_groups(G, dtype, causal):
    """RoPE append at every group size the kernel is built for (a tile's 128
    rows are 128 / G tokens of G heads) in both 16-bit types; the requests
    span several tiles, a ragged last tile and a split segment."""
    say(f"[case] rope append G={G} {dtype} causal={causal}")
    w = wl.small_append(380 + G, [5, 130 // G + 3, 300], [40, 260, 900], 16, 2 * G, 2,
                        dtype=dtype, causal=causal)
    w.rope_theta = 500000.0
    o_ref, l_ref = ora.append_workload(w)
    o, l = run_append(w, num_workers=9)
    assert_parity(o, l, o_ref, l_ref, dtype, what=f"rope append G{G} {dtype}")


def test_rope_append_many_way_splits():
    """RoPE append with tiles split over more than 4 workers, so the plan merge
    kernel (not the in-kernel merge) combines the 128-row partial states; the
    plan's mode is checked."""
    import torch
    say("[case] rope append, many-way splits")
    w = wl.small_append(391, [40, 128, 7], [2000, 1500, 900], 16, 8, 2, causal=True)
    w.rope_theta = 500000.0
    kv = w.kv
    dev = upload_kv(kv)
    q = wl.to_torch(w.q, "bf16", "cuda")
    params = abp.make_params(8, 2, 128, 16, torch.bfloat16, causal=True, rope_theta=w.rope_theta)
    app = abp.BatchAppend(params, max_batch=3, max_qo_tokens=256, num_workers=96)
    plan = app.plan(w.qo_indptr, kv.kv_indptr, kv.kv_last_page_len)
    torch.cuda.synchronize()
    arr = abp.decode_plan_arrays(app.host_ws.numpy(), plan)
    assert int(arr["merge_kernel"][0]) == 1 and int(arr["tile_num_partials"].max()) > 4
    o, lse = app.run(q, dev["k"], dev["v"], i32(w.qo_indptr), dev["indptr"], dev["indices"],
                     dev["lpl"])
    torch.cuda.synchronize()
    o_ref, l_ref = ora.append_workload(w)
    assert_parity(o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, l_ref, "bf16",
                  what="rope append, many-way splits")


@pytest.mark.parametrize("P", [3, 256])
def test_rope_append_page_sizes(P):
    """RoPE append on the per-token page path (P = 3) and with large pages."""
    w = wl.small_append(370 + P, [5, 64, 150], [70, 64, 600], P, 8, 2, causal=True)
    w.rope_theta = 500000.0
    o_ref, l_ref = ora.append_workload(w)
    o, l = run_append(w, num_workers=10)
    assert_parity(o, l, o_ref, l_ref, "bf16", what=f"rope append P{P}")


# ----------------------------------------------------------------------------
# cascade / composable formats
# ----------------------------------------------------------------------------
def run_cascade(w, num_workers=0, prefix_workers=0):
    import torch
    pre, kv = w.prefix, w.kv
    cas = abp.CascadeDecode(w.num_qo_heads, w.num_kv_heads, w.head_dim, pre.page_size,
                            kv.page_size, torch.bfloat16 if w.dtype == "bf16" else torch.float16,
                            max_batch=w.batch, rope_theta=w.rope_theta, num_workers=num_workers,
                            prefix_workers=prefix_workers)
    cas.plan(w.batch, pre.kv_indptr, pre.kv_last_page_len, kv.kv_indptr, kv.kv_last_page_len)
    dp, ds = upload_kv(pre), upload_kv(kv)
    q = wl.to_torch(w.q, w.dtype, "cuda")
    o, l = cas.run(q, dp["k"], dp["v"], i32([0, w.batch]), dp["indptr"], dp["indices"], dp["lpl"],
                   ds["k"], ds["v"], ds["indptr"], ds["indices"], ds["lpl"],
                   q_pos=i32(w.q_pos), kv_pos_offset=i32(w.kv_pos_offset))
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), l.cpu().numpy()


def small_cascade(seed, theta):
    rng = np.random.Generator(np.random.PCG64(seed))
    B, pre_len = 5, 700
    prefix = wl.make_paged_kv(rng, np.array([pre_len]), 256, 2, 128, "bf16", extra_pages=1)
    suf = rng.integers(1, 300, size=B)
    kv = wl.make_paged_kv(rng, suf, 16, 2, 128, "bf16", extra_pages=3)
    q = wl.normal_bits(rng, (B, 8, 128), "bf16")
    w = wl.Workload("small_cascade", "cascade", seed, "bf16", 8, 2, 128, kv, q,
                    rope_theta=theta, prefix=prefix)
    if theta:
        w.kv_pos_offset = np.full(B, pre_len, np.int32)
        w.q_pos = (pre_len + suf - 1).astype(np.int32)
    return w


@pytest.mark.parametrize("theta", [0.0, 500000.0])
def test_small_cascade_parity(theta):
    w = small_cascade(350, theta)
    o_ref, l_ref = ora.decode_workload(w)
    o, l = run_cascade(w, num_workers=9, prefix_workers=4)
    assert_parity(o, l, o_ref, l_ref, "bf16", what=f"cascade theta={theta}")


def test_cascade_rope_full():
    """64 requests sharing an 8192-token prefix (pages of 256) plus suffixes of
    256..1024 tokens (pages of 16), GQA 32/8, bf16, RoPE theta 500000, in the
    default launch configuration; every request compared."""
    w = wl.cascade_rope()
    say(f"[case] {w.name}")
    o, l = run_cascade(w)
    o_ref, l_ref = ora.decode_workload(w)
    assert_parity(o, l, o_ref, l_ref, "bf16", what="cascade rope, all requests")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))


def cascade_case(seed, B, hkv, G, theta, dtype="bf16", pre_len=900, zero_suffix=True):
    rng = np.random.Generator(np.random.PCG64(seed))
    prefix = wl.make_paged_kv(rng, np.array([pre_len]), 256, hkv, 128, dtype, extra_pages=1)
    suf = rng.integers(1, 200, size=B)
    if zero_suffix:
        suf[B // 3] = 0
    kv = wl.make_paged_kv(rng, suf, 16, hkv, 128, dtype, extra_pages=3)
    q = wl.normal_bits(rng, (B, hkv * G, 128), dtype)
    w = wl.Workload("cascade_case", "cascade", seed, dtype, hkv * G, hkv, 128, kv, q,
                    rope_theta=theta, prefix=prefix)
    if theta:
        w.kv_pos_offset = np.full(B, pre_len, np.int32)
        w.q_pos = (pre_len + np.maximum(suf, 1) - 1).astype(np.int32)
    return w


@pytest.mark.parametrize("theta", [0.0, 500000.0])
@pytest.mark.parametrize("pw,sw", [(1, 1), (3, 7), (0, 0), (40, 300)])
def test_cascade_single_call_shapes(theta, pw, sw):
    """abp_cascade_run over query tiles that do not divide the batch (100
    queries: 64-query tiles without RoPE, 32 with), 8 kv heads (4-head decode
    tiles on the matrix cores), a suffix of length 0, and worker counts that
    leave the prefix tiles unsplit (1), merged inside the append kernel (3),
    or split over many partials (default, 40), and the suffix tiles unsplit,
    split a few ways or many."""
    w = cascade_case(700 + pw + sw, 100, 8, 4, theta)
    say(f"[case] cascade B=100 hkv=8 G=4 theta={theta} prefix W{pw} suffix W{sw}")
    o_ref, l_ref = ora.decode_workload(w)
    o, l = run_cascade(w, num_workers=sw, prefix_workers=pw)
    assert_parity(o, l, o_ref, l_ref, "bf16", what=f"cascade theta={theta} W{pw}/{sw}")


def test_cascade_single_call_group8_fp16():
    """G = 8 (64 qo heads over 8 kv heads), fp16, RoPE."""
    w = cascade_case(760, 37, 8, 8, 500000.0, dtype="fp16")
    o_ref, l_ref = ora.decode_workload(w)
    o, l = run_cascade(w, num_workers=11, prefix_workers=6)
    assert_parity(o, l, o_ref, l_ref, "fp16", what="cascade G8 fp16")
