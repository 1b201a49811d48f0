"""C-ABI checks that need no GPU: exports, status codes, validation, and the
C++ planner against the reference planner (bit-exact)."""
import ctypes
import os
import re

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import attention_bsr_paged_amd as abp
from oracle.plan_ref import KIND_APPEND, KIND_DECODE, plan_ref

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "abp.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(abp_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), f"{n} declared in abp.h but not exported"
    assert set(names) == set(abp.EXPORTED_SYMBOLS)


def test_status_strings(lib):
    assert abp.abp_status_string(0) == "ok"
    for s in (-1, -2, -3, -4, -5):
        assert abp.abp_status_string(s) not in ("ok", "unknown status")
    assert abp.abp_status_string(42) == "unknown status"


def P(**kw):
    base = dict(num_qo_heads=32, num_kv_heads=8, head_dim=128, page_size=16, dtype="bf16")
    base.update(kw)
    return abp.make_params(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=64), abp.ABP_ERR_UNSUPPORTED),
    (dict(num_qo_heads=30), abp.ABP_ERR_INVALID_ARG),
    (dict(num_qo_heads=24), abp.ABP_ERR_UNSUPPORTED),      # group 3
    (dict(page_size=0), abp.ABP_ERR_INVALID_ARG),
    (dict(num_qo_heads=32, num_kv_heads=2), abp.ABP_ERR_UNSUPPORTED),  # decode group 16
])
def test_param_validation(lib, kw, status):
    with pytest.raises(abp.AbpError) as e:
        abp.abp_workspace_size(abp.ABP_KIND_DECODE, P(**kw), 4, 0, 8)
    assert e.value.status == status


def test_bad_dtype(lib):
    p = P()
    p.qkv_dtype = abp.ABP_F32
    with pytest.raises(abp.AbpError) as e:
        abp.abp_workspace_size(abp.ABP_KIND_DECODE, p, 4, 0, 8)
    assert e.value.status == abp.ABP_ERR_UNSUPPORTED


def _ws(kind, p, max_batch, max_qo, W):
    h, _ = abp.abp_workspace_size(kind, p, max_batch, max_qo, W)
    return np.zeros(h, np.uint8)


@pytest.mark.parametrize("indptr,lpl,status", [
    ([0, 2, 1], [1, 1], abp.ABP_ERR_INVALID_ARG),
    ([1, 2, 3], [1, 1], abp.ABP_ERR_INVALID_ARG),
    ([0, 1, 2], [0, 1], abp.ABP_ERR_INVALID_ARG),
    ([0, 1, 2], [1, 17], abp.ABP_ERR_INVALID_ARG),
])
def test_index_validation(lib, indptr, lpl, status):
    p = P()
    with pytest.raises(abp.AbpError) as e:
        abp.abp_plan_host(abp.ABP_KIND_DECODE, p, 2, None, indptr, lpl, 2, 0, 8,
                          _ws(0, p, 2, 0, 8))
    assert e.value.status == status


def test_workspace_and_capacity_errors(lib):
    p = P()
    ws = _ws(0, p, 2, 0, 8)
    with pytest.raises(abp.AbpError) as e:        # batch above max_batch
        abp.abp_plan_host(0, p, 3, None, [0, 1, 2, 3], [1, 1, 1], 2, 0, 8, ws)
    assert e.value.status == abp.ABP_ERR_WORKSPACE_TOO_SMALL
    with pytest.raises(abp.AbpError) as e:        # host workspace too small
        abp.abp_plan_host(0, p, 2, None, [0, 1, 2], [1, 1], 2, 0, 8, ws[:64])
    assert e.value.status == abp.ABP_ERR_WORKSPACE_TOO_SMALL
    pa = P(causal=True)
    wa = _ws(1, pa, 1, 8, 8)
    with pytest.raises(abp.AbpError) as e:        # causal with qo_len > kv_len
        abp.abp_plan_host(1, pa, 1, [0, 8], [0, 1], [4], 1, 8, 8, wa)
    assert e.value.status == abp.ABP_ERR_INVALID_ARG
    with pytest.raises(abp.AbpError) as e:        # more query tokens than planned for
        abp.abp_plan_host(1, pa, 1, [0, 9], [0, 1], [16], 1, 8, 8, wa)
    assert e.value.status == abp.ABP_ERR_WORKSPACE_TOO_SMALL


def test_run_rejects_mismatched_params_before_any_launch(lib):
    """The fingerprint check fails on the host, so no device is touched."""
    p = P()
    ws = _ws(0, p, 2, 0, 8)
    plan = abp.abp_plan_host(0, p, 2, None, [0, 1, 2], [3, 4], 2, 0, 8, ws)
    other = P(page_size=32)
    st_ = lib.abp_decode_run(ctypes.byref(plan), ctypes.byref(other), *([None] * 10), None, 0, None)
    assert st_ == abp.ABP_ERR_PLAN_MISMATCH
    plan.kind = abp.ABP_KIND_APPEND
    st_ = lib.abp_decode_run(ctypes.byref(plan), ctypes.byref(p), *([None] * 10), None, 0, None)
    assert st_ == abp.ABP_ERR_PLAN_MISMATCH


def _compare(kind, p, B, qo_indptr, kv_indptr, lpl, W, G, max_qo=0):
    ws = _ws(kind, p, B, max_qo, W)
    plan = abp.abp_plan_host(kind, p, B, qo_indptr, kv_indptr, lpl, B, max_qo, W, ws)
    got = abp.decode_plan_arrays(ws, plan)
    no_split = W == abp.ABP_WORKERS_PER_TILE
    if no_split:
        W = plan.num_workers   # the tile capacity
        assert W == max(1, plan.max_tiles)
    if kind == KIND_DECODE:
        # decode tiles take 4 consecutive kv heads when the count allows, else 1
        hpt = 4 if p.num_kv_heads % 4 == 0 else 1
        assert int(got["tile_heads"][0]) == hpt
        assert plan.rows_per_tile == hpt * G
        ref = plan_ref(KIND_DECODE, B, kv_indptr, lpl, p.page_size, p.num_kv_heads, W, 64,
                       heads_per_tile=hpt, no_split=no_split)
    else:
        ref = plan_ref(KIND_APPEND, B, kv_indptr, lpl, p.page_size, p.num_kv_heads, W, 64,
                       qo_indptr=qo_indptr, tile_q=plan.rows_per_tile // G,
                       causal=bool(p.causal),
                       no_split=no_split)
    for k, v in ref.items():
        assert np.array_equal(got[k], v), k
    # merge placement: decode always uses the merge kernel; append merges inside
    # the kernel unless some tile has more than 4 partials
    np_max = int(ref["tile_num_partials"].max()) if len(ref["tile_num_partials"]) else 0
    expect = 1 if kind == KIND_DECODE or np_max > 4 else 0
    assert int(got["merge_kernel"][0]) == expect
    assert plan.num_segments == len(ref["seg_tile"])
    assert plan.num_merges == len(ref["merge_list"])


@settings(max_examples=120, deadline=None)
@given(st.data())
def test_cpp_planner_matches_reference(data):
    abp.load_library()
    B = data.draw(st.integers(0, 12))
    page = data.draw(st.sampled_from([1, 3, 16, 256]))
    G = data.draw(st.sampled_from([1, 2, 4, 8]))
    hkv = data.draw(st.sampled_from([1, 2, 3, 4, 8, 12, 16]))
    W = data.draw(st.sampled_from([abp.ABP_WORKERS_PER_TILE]) | st.integers(1, 70))
    kv_len = data.draw(st.lists(st.integers(0, 3000), min_size=B, max_size=B))
    npg = [-(-n // page) for n in kv_len]
    indptr = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
    lpl = np.array([n - (k - 1) * page if k else 0 for n, k in zip(kv_len, npg)], np.int32)
    if data.draw(st.booleans()):
        p = P(num_qo_heads=hkv * G, num_kv_heads=hkv, page_size=page)
        _compare(KIND_DECODE, p, B, None, indptr, lpl, W, G)
    else:
        causal = data.draw(st.booleans())
        qo = [data.draw(st.integers(0, min(n, 300) if causal else 300)) for n in kv_len]
        qo_indptr = np.concatenate([[0], np.cumsum(qo)]).astype(np.int32)
        p = P(num_qo_heads=hkv * G, num_kv_heads=hkv, page_size=page, causal=causal)
        _compare(KIND_APPEND, p, B, qo_indptr, indptr, lpl, W, G, max_qo=int(qo_indptr[-1]))


@pytest.mark.parametrize("name", ["batch_decode", "skewed_decode"])
def test_planner_on_named_decode_workloads(lib, name):
    """The planner on the named workloads' page tables (lengths only, no values)."""
    from attention_bsr_paged_amd import workloads as wl
    rng = np.random.Generator(np.random.PCG64(1002 if name == "batch_decode" else 1003))
    if name == "batch_decode":
        kv_len = rng.integers(512, 4096, size=64, endpoint=True)
    else:
        rest = np.clip(np.rint(np.exp(rng.normal(np.log(512.0), 1.0, size=127))), 16, 16384)
        kv_len = np.concatenate([[32768], rest]).astype(np.int64)
    indptr, _, lpl = wl.page_table(kv_len, 16, np.arange(10 ** 6))
    for W in (256, 512, 1024, abp.ABP_WORKERS_PER_TILE):
        _compare(KIND_DECODE, P(), len(kv_len), None, indptr, lpl, W, 4)


@pytest.mark.parametrize("rope", [0, 1])
def test_planner_on_ragged_append(lib, rope):
    """The ragged causal append's page table (lengths only) at worker counts
    that co-schedule 8, 4 and 2 query tiles and at one that does not."""
    from attention_bsr_paged_amd import workloads as wl
    rng = np.random.Generator(np.random.PCG64(1004))
    qo_len = rng.integers(128, 1024, size=16, endpoint=True)
    kv_len = rng.integers(1024, 8192, size=16, endpoint=True) + qo_len
    qo_indptr = np.concatenate([[0], np.cumsum(qo_len)]).astype(np.int32)
    indptr, _, lpl = wl.page_table(kv_len, 16, np.arange(10 ** 6))
    p = P(causal=True, rope_theta=5e5 if rope else 0.0)
    for W in (256, 224, 208, 200):
        _compare(KIND_APPEND, p, 16, qo_indptr, indptr, lpl, W, 4, max_qo=int(qo_indptr[-1]))


# ----------------------------------------------------------------------------
# block-sparse plans, LLaMA 3.1 frequency table, page append argument checks
# ----------------------------------------------------------------------------
@settings(max_examples=60, deadline=None)
@given(st.data())
def test_bsr_plan_matches_reference_over_row_blocks(data):
    """A block-sparse plan is the append plan of its row blocks (queries
    [i R, min((i+1) R, M)), pages = listed column blocks, all full)."""
    abp.load_library()
    C = data.draw(st.sampled_from([1, 3, 16, 64]))
    R = data.draw(st.sampled_from([1, 5, 16, 64, 100]))
    G = data.draw(st.sampled_from([1, 4, 8]))
    hkv = data.draw(st.sampled_from([1, 2, 8]))
    W = data.draw(st.integers(1, 70))
    ncb = data.draw(st.integers(0, 40))
    M = data.draw(st.integers(0, 700))
    nrb = -(-M // R)
    counts = [data.draw(st.integers(0, ncb)) for _ in range(nrb)]
    indptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    p = P(num_qo_heads=hkv * G, num_kv_heads=hkv, page_size=C)
    h, _ = abp.abp_workspace_size(abp.ABP_KIND_BSR, p, nrb, M, W)
    ws = np.zeros(h, np.uint8)
    plan = abp.abp_bsr_plan_host(p, M, ncb * C, R, indptr, nrb, M, W, ws)
    assert plan.kind == abp.ABP_KIND_BSR
    got = abp.decode_plan_arrays(ws, plan)
    qo_indptr = np.minimum(np.arange(nrb + 1) * R, M)
    ref = plan_ref(KIND_APPEND, nrb, indptr, np.full(nrb, C), C, hkv, W, 64,
                   qo_indptr=qo_indptr, tile_q=256 // G, causal=False, lanes=1)
    for k, v in ref.items():
        assert np.array_equal(got[k], v), k
    # the derived query ranges and page counts the run reads from the blob
    b = ws.view(np.int32)
    aux = got["off_aux"]
    cap = (len(b) - aux) // 2
    assert np.array_equal(b[aux:aux + nrb + 1], qo_indptr)
    lpl_at = aux + ((plan.max_tiles // hkv + 1 + 3) & ~3)
    assert np.all(b[lpl_at:lpl_at + nrb] == C)
    assert cap >= nrb


def test_bsr_plan_validation(lib):
    p = P(page_size=16)
    h, _ = abp.abp_workspace_size(abp.ABP_KIND_BSR, p, 4, 256, 8)
    ws = np.zeros(h, np.uint8)
    for args, status in [
        ((256, 100, 64, [0, 1, 2, 3, 4]), abp.ABP_ERR_INVALID_ARG),      # N % C != 0
        ((256, 128, 64, [0, 1, 2, 1, 4]), abp.ABP_ERR_INVALID_ARG),      # decreasing indptr
        ((256, 128, 64, [1, 1, 2, 3, 4]), abp.ABP_ERR_INVALID_ARG),      # indptr[0] != 0
        ((256, 128, 64, [0, 9, 9, 9, 9]), abp.ABP_ERR_INVALID_ARG),      # 9 > N / C blocks
        ((320, 128, 64, [0] * 6), abp.ABP_ERR_WORKSPACE_TOO_SMALL),      # M > max_M
        ((256, 128, 32, [0] * 9), abp.ABP_ERR_WORKSPACE_TOO_SMALL),      # 8 row blocks > 4
    ]:
        with pytest.raises(abp.AbpError) as e:
            abp.abp_bsr_plan_host(p, *args, 4, 256, 8, ws)
        assert e.value.status == status, args
    for bad in (P(causal=True), P(rope_theta=1e4)):
        with pytest.raises(abp.AbpError) as e:
            abp.abp_workspace_size(abp.ABP_KIND_BSR, bad, 4, 256, 8)
        assert e.value.status == abp.ABP_ERR_UNSUPPORTED
    with pytest.raises(abp.AbpError):              # the generic planner refuses BSR plans
        abp.abp_plan_host(abp.ABP_KIND_BSR, p, 1, [0, 4], [0, 1], [16], 1, 4, 8, ws)


@pytest.mark.parametrize("l31", [None, abp.LLAMA31_ROPE, (4.0, 2.0, 8.0, 4096.0)])
def test_rope_frequency_table_matches_oracle(lib, l31):
    """The host table (revolutions per position, fp32 hi + lo) against the
    oracle's float64 frequencies, LLaMA 3.1-scaled or not."""
    from oracle import attention as ora
    p = P(rope_theta=500000.0, rope_llama31=l31)
    ws = _ws(0, p, 2, 0, 8)
    plan = abp.abp_plan_host(0, p, 2, None, [0, 1, 2], [3, 4], 2, 0, 8, ws)
    t = abp.decode_plan_arrays(ws, plan)["rope"].astype(np.float64)
    rev = t[0::2] + t[1::2]
    want = ora.rope_inv_freq(128, 500000.0, l31) / (2 * np.pi)
    assert np.max(np.abs(rev - want) / want) < 1e-13


def test_llama31_params_validated(lib):
    for bad in [(8.0, 1.0, 1.0, 8192.0), (0.0, 1.0, 4.0, 8192.0), (8.0, 1.0, 4.0, 0.0)]:
        with pytest.raises(abp.AbpError) as e:
            abp.abp_workspace_size(0, P(rope_theta=5e5, rope_llama31=bad), 2, 0, 8)
        assert e.value.status == abp.ABP_ERR_INVALID_ARG


def test_page_append_argument_checks(lib):
    p = P()
    # nothing to write: returns before touching any device
    assert lib.abp_append_paged_kv(ctypes.byref(p), 3, 0, *([None] * 8), None) == abp.ABP_OK
    assert lib.abp_append_paged_kv(ctypes.byref(p), 0, 5, *([None] * 8), None) == abp.ABP_OK
    assert lib.abp_append_paged_kv(ctypes.byref(p), 2, 4, *([None] * 8), None) == \
        abp.ABP_ERR_INVALID_ARG
    assert lib.abp_append_paged_kv(ctypes.byref(p), -1, 4, *([None] * 8), None) == \
        abp.ABP_ERR_INVALID_ARG
    q = P(head_dim=64)
    assert lib.abp_append_paged_kv(ctypes.byref(q), 2, 4, *([None] * 8), None) == \
        abp.ABP_ERR_UNSUPPORTED


def test_fp8_kv_params(lib):
    ok = P(kv_fp8=True, k_scale=0.5, v_scale=2.0)
    abp.abp_workspace_size(abp.ABP_KIND_DECODE, ok, 4, 0, 8)
    for kind, bad, status in [
        (abp.ABP_KIND_APPEND, P(kv_fp8=True), abp.ABP_ERR_UNSUPPORTED),
        (abp.ABP_KIND_BSR, P(kv_fp8=True), abp.ABP_ERR_UNSUPPORTED),
        (abp.ABP_KIND_DECODE, P(kv_fp8=True, rope_theta=1e4), abp.ABP_ERR_UNSUPPORTED),
        (abp.ABP_KIND_DECODE, P(kv_fp8=True, k_scale=0.0), abp.ABP_ERR_INVALID_ARG),
    ]:
        with pytest.raises(abp.AbpError) as e:
            abp.abp_workspace_size(kind, bad, 4, 16, 8)
        assert e.value.status == status
    # the scales enter the plan fingerprint: a run with other scales is refused
    ws = _ws(0, ok, 2, 0, 8)
    plan = abp.abp_plan_host(0, ok, 2, None, [0, 1, 2], [3, 4], 2, 0, 8, ws)
    other = P(kv_fp8=True, k_scale=0.5, v_scale=1.0)
    st_ = lib.abp_decode_run(ctypes.byref(plan), ctypes.byref(other), *([None] * 10), None, 0, None)
    assert st_ == abp.ABP_ERR_PLAN_MISMATCH


def test_rope_interleave_param(lib):
    p = P(rope_theta=5e5, rope_interleave=True)
    ws = _ws(0, p, 2, 0, 8)
    plan = abp.abp_plan_host(0, p, 2, None, [0, 1, 2], [3, 4], 2, 0, 8, ws)
    # the pairing enters the fingerprint: a run with the other pairing is refused
    other = P(rope_theta=5e5)
    st_ = lib.abp_decode_run(ctypes.byref(plan), ctypes.byref(other), *([None] * 10), None, 0, None)
    assert st_ == abp.ABP_ERR_PLAN_MISMATCH
    bad = P(rope_theta=5e5)
    bad.rope_interleave = 2
    with pytest.raises(abp.AbpError) as e:
        abp.abp_workspace_size(0, bad, 2, 0, 8)
    assert e.value.status == abp.ABP_ERR_INVALID_ARG


# ----------------------------------------------------------------------------
# mixed decode + append batches (one plan, two sub-plans)
# ----------------------------------------------------------------------------
def _pod_ws(p, md, ma, mq, groups):
    h, _ = abp.abp_pod_workspace_size(p, md, ma, mq, groups)
    return np.zeros(h, np.uint8)


def _pod_case(rng, B, P_, causal):
    kv_len = rng.integers(0 if not causal else 1, 3000, size=B)
    pages = (kv_len + P_ - 1) // P_
    indptr = np.concatenate([[0], np.cumsum(pages)]).astype(np.int32)
    lpl = np.where(pages > 0, kv_len - (pages - 1) * P_, 1).astype(np.int32)
    return kv_len, indptr, lpl


@pytest.mark.parametrize("groups,decode_groups", [(256, 0), (256, 40), (16, 0), (2, 0), (9, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_pod_subplans_match_reference(lib, groups, decode_groups, causal):
    """Each sub-plan is the reference plan of its part with the split's worker counts."""
    rng = np.random.default_rng(groups + decode_groups + causal)
    p = P(causal=causal)
    _, d_indptr, d_lpl = _pod_case(rng, 9, 16, False)
    a_len, a_indptr, a_lpl = _pod_case(rng, 5, 16, True)
    qo_len = np.minimum(rng.integers(1, 600, size=5), a_len)
    qo = np.concatenate([[0], np.cumsum(qo_len)]).astype(np.int32)
    ws = _pod_ws(p, 9, 5, int(qo[-1]), groups)
    plan = abp.abp_pod_plan_host(p, d_indptr, d_lpl, qo, a_indptr, a_lpl, 9, 5, int(qo[-1]),
                                 groups, decode_groups, ws)
    wd, wa = plan.decode.num_workers, plan.append.num_workers
    assert plan.num_groups == groups and wd + wa == groups and wd >= 1 and wa >= 1
    if decode_groups:
        assert wd == decode_groups
    elif groups >= 16:
        assert wd % 8 == 0
    dblob = ws[plan.decode_host_offset:plan.append_host_offset]
    ablob = ws[plan.append_host_offset:]
    got_d = abp.decode_plan_arrays(dblob, plan.decode)
    ref_d = plan_ref(KIND_DECODE, 9, d_indptr, d_lpl, 16, 8, wd, 64, heads_per_tile=4)
    for k, v in ref_d.items():
        assert np.array_equal(got_d[k], v), k
    got_a = abp.decode_plan_arrays(ablob, plan.append)
    ref_a = plan_ref(KIND_APPEND, 5, a_indptr, a_lpl, 16, 8, wa, 64, qo_indptr=qo,
                     tile_q=256 // 4, causal=causal)
    for k, v in ref_a.items():
        assert np.array_equal(got_a[k], v), k
    assert int(got_d["merge_kernel"][0]) == 1


def test_pod_split_follows_the_work(lib):
    """More decode bytes against the same append work gets more decode groups;
    a part with no request gets no group."""
    p = P(causal=True)
    qo = np.array([0, 512], np.int32)
    a_indptr, a_lpl = np.array([0, 160], np.int32), np.array([16], np.int32)
    splits = []
    for n in (4, 64, 512):
        d_indptr = (np.arange(n + 1) * 128).astype(np.int32)   # 2048 tokens each
        d_lpl = np.full(n, 16, np.int32)
        ws = _pod_ws(p, n, 1, 512, 256)
        plan = abp.abp_pod_plan_host(p, d_indptr, d_lpl, qo, a_indptr, a_lpl, n, 1, 512, 256,
                                     0, ws)
        splits.append(plan.decode.num_workers)
    assert splits[0] < splits[1] < splits[2] <= 248, splits
    ws = _pod_ws(p, 4, 1, 512, 256)
    only_a = abp.abp_pod_plan_host(p, None, None, qo, a_indptr, a_lpl, 4, 1, 512, 256, 0, ws)
    assert (only_a.decode.num_workers, only_a.append.num_workers) == (0, 256)
    only_d = abp.abp_pod_plan_host(p, [0, 1], [5], None, None, None, 4, 1, 512, 256, 0, ws)
    assert (only_d.decode.num_workers, only_d.append.num_workers) == (256, 0)


@pytest.mark.parametrize("kw", [dict(rope_theta=1e4), dict(page_size=8), dict(num_qo_heads=16),
                                dict(num_kv_heads=2, num_qo_heads=8),
                                dict(kv_fp8=True, k_scale=1.0, v_scale=1.0)])
def test_pod_rejects_unsupported_params(lib, kw):
    with pytest.raises(abp.AbpError) as e:
        abp.abp_pod_workspace_size(P(**kw), 4, 4, 64, 256)
    assert e.value.status == abp.ABP_ERR_UNSUPPORTED


def test_pod_plan_errors(lib):
    p = P()
    ws = _pod_ws(p, 2, 1, 8, 256)
    qo = np.array([0, 4], np.int32)
    with pytest.raises(abp.AbpError) as e:      # more decode requests than planned for
        abp.abp_pod_plan_host(p, [0, 1, 2, 3], [1, 1, 1], qo, [0, 1], [4], 2, 1, 8, 256, 0, ws)
    assert e.value.status == abp.ABP_ERR_WORKSPACE_TOO_SMALL
    with pytest.raises(abp.AbpError) as e:      # host workspace too small
        abp.abp_pod_plan_host(p, [0, 1], [1], qo, [0, 1], [4], 2, 1, 8, 256, 0, ws[:100])
    assert e.value.status == abp.ABP_ERR_WORKSPACE_TOO_SMALL
    with pytest.raises(abp.AbpError) as e:      # a bad decode page table
        abp.abp_pod_plan_host(p, [0, 1], [0], qo, [0, 1], [4], 2, 1, 8, 256, 0, ws)
    assert e.value.status == abp.ABP_ERR_INVALID_ARG
    with pytest.raises(abp.AbpError) as e:      # one workgroup cannot hold both roles
        abp.abp_pod_workspace_size(p, 2, 1, 8, 1)
    assert e.value.status == abp.ABP_ERR_INVALID_ARG


def test_missing_library_fails_loudly(tmp_path):
    """The product path has no fallback: a missing library is an error."""
    with pytest.raises(RuntimeError, match="no fallback"):
        abp.load_library(str(tmp_path / "libabp.so"))


def test_product_code_does_not_reach_the_oracle():
    """Nothing in the package imports the oracle (it is test infrastructure)."""
    pkg = os.path.join(os.path.dirname(os.path.dirname(__file__)), "attention_bsr_paged_amd")
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(root, f), encoding="utf-8").read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), f
                assert "oracle/" not in text, f


def test_decode_static_rejects_batches_beyond_its_arrays(lib):
    """The no-allocation decode refuses a batch whose plan exceeds its static
    host array before any GPU work (explicit worker count: no device query)."""
    import ctypes
    import torch
    p = abp.make_params(32, 8, 128, 16, torch.bfloat16)
    B = 20000
    indptr = np.arange(B + 1, dtype=np.int32)
    lpl = np.ones(B, np.int32)
    st = lib.abp_decode_static(ctypes.byref(p), B, indptr.ctypes.data, lpl.ctypes.data, 256,
                               *([None] * 10), None)
    assert st == abp.ABP_ERR_WORKSPACE_TOO_SMALL
    msg = abp.abp_last_error()
    assert "abp_decode_static" in msg and str(abp.ABP_STATIC_PLAN_BYTES) in msg
    # too many workers for the device array
    st = lib.abp_decode_static(ctypes.byref(p), 4, indptr[:5].ctypes.data, lpl.ctypes.data,
                               4096, *([None] * 10), None)
    assert st == abp.ABP_ERR_WORKSPACE_TOO_SMALL
    assert str(abp.ABP_STATIC_SCRATCH_BYTES) in abp.abp_last_error()


def test_pages_of_2gib_or_more_are_refused(lib):
    import ctypes
    import torch
    hb, db = ctypes.c_size_t(), ctypes.c_size_t()
    ok = abp.make_params(32, 8, 128, 1 << 19, torch.bfloat16)        # 1 GiB pages
    assert lib.abp_workspace_size(0, ctypes.byref(ok), 4, 0, 16, ctypes.byref(hb),
                                  ctypes.byref(db)) == abp.ABP_OK
    big = abp.make_params(32, 8, 128, 1 << 20, torch.bfloat16)       # 2 GiB pages
    assert lib.abp_workspace_size(0, ctypes.byref(big), 4, 0, 16, ctypes.byref(hb),
                                  ctypes.byref(db)) == abp.ABP_ERR_UNSUPPORTED
    assert "2 GiB" in abp.abp_last_error()


def test_cascade_run_checks_its_plans(lib):
    """abp_cascade_run refuses, on the host and before any launch, a prefix
    plan whose query tiles do not cover the suffix batch, a causal prefix,
    level params that do not write fp32 states, swapped plans and a bad output
    dtype (the prefix's exact query count is the caller's contract: the plan
    does not hold it)."""
    B = 6
    pre_p = P(page_size=256, out_dtype="fp32")
    suf_p = P(out_dtype="fp32")
    pws = _ws(abp.ABP_KIND_APPEND, pre_p, 1, B, 8)
    pre = abp.abp_plan_host(abp.ABP_KIND_APPEND, pre_p, 1, [0, B], [0, 2], [256], 1, B, 8, pws)
    sws = _ws(abp.ABP_KIND_DECODE, suf_p, B, 0, 8)
    indptr = np.arange(B + 1, dtype=np.int32) * 3
    suf = abp.abp_plan_host(abp.ABP_KIND_DECODE, suf_p, B, None, indptr, np.full(B, 5, np.int32),
                            B, 0, 8, sws)
    fake_ws, big = 1 << 20, 1 << 40   # never dereferenced: every case fails before a launch

    def run(pp, pre_params, sp, suf_params, out=abp.ABP_BF16):
        return lib.abp_cascade_run(ctypes.byref(pp), ctypes.byref(pre_params), fake_ws, big,
                                   ctypes.byref(sp), ctypes.byref(suf_params), fake_ws, big,
                                   *([None] * 20), out, None)

    assert run(pre, pre_p, suf, P()) == abp.ABP_ERR_PLAN_MISMATCH  # params differ from the plan
    bf_p = P(out_dtype="bf16")
    sws2 = _ws(abp.ABP_KIND_DECODE, bf_p, B, 0, 8)
    suf_bf = abp.abp_plan_host(abp.ABP_KIND_DECODE, bf_p, B, None, indptr,
                               np.full(B, 5, np.int32), B, 0, 8, sws2)
    assert run(pre, pre_p, suf_bf, bf_p) == abp.ABP_ERR_UNSUPPORTED  # level states must be fp32
    # a prefix over fewer query tiles than the suffix batch needs (64 queries per tile)
    B2 = 70
    indptr2 = np.arange(B2 + 1, dtype=np.int32) * 3
    sws3 = _ws(abp.ABP_KIND_DECODE, suf_p, B2, 0, 8)
    suf2 = abp.abp_plan_host(abp.ABP_KIND_DECODE, suf_p, B2, None, indptr2,
                             np.full(B2, 5, np.int32), B2, 0, 8, sws3)
    assert run(pre, pre_p, suf2, suf_p) == abp.ABP_ERR_PLAN_MISMATCH
    # a well-formed pair gets past the plan checks to the tensor checks
    assert run(pre, pre_p, suf, suf_p) == abp.ABP_ERR_INVALID_ARG
    causal_p = P(page_size=256, out_dtype="fp32", causal=True)
    cws = _ws(abp.ABP_KIND_APPEND, causal_p, 1, B, 8)
    cpre = abp.abp_plan_host(abp.ABP_KIND_APPEND, causal_p, 1, [0, B], [0, 2], [256], 1, B, 8,
                             cws)
    assert run(cpre, causal_p, suf, suf_p) == abp.ABP_ERR_PLAN_MISMATCH
    assert run(suf, suf_p, pre, pre_p) == abp.ABP_ERR_PLAN_MISMATCH  # swapped kinds
    assert run(pre, pre_p, suf, suf_p, out=abp.ABP_F32 + 7) == abp.ABP_ERR_UNSUPPORTED
