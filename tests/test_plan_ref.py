"""Pins of the reference planner: hand-derived plans and the Stream-K invariants (CPU)."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.plan_ref import KIND_APPEND, KIND_DECODE, PlanError, co_lanes, plan_ref


def test_decode_hand_example():
    # page 4; request 0 owns 3 pages with 2 valid slots in the last (10 tokens),
    # request 1 owns 1 full page (4 tokens). tile_kv 4: tile 0 costs 3 blocks, tile 1
    # costs 1; N = 4, W = 3 -> quota 2. Worker 0: blocks 0-1 = tile 0 keys [0, 8).
    # Worker 1: block 2 = tile 0 keys [8, 10), block 3 = tile 1 keys [0, 4). Worker 2: none.
    p = plan_ref(KIND_DECODE, 2, [0, 3, 4], [2, 4], 4, 1, 3, 4)
    assert p["quota"].tolist() == [2]
    assert p["worker_seg_indptr"].tolist() == [0, 1, 3, 3]
    assert p["seg_tile"].tolist() == [0, 0, 1]
    assert p["seg_kv_begin"].tolist() == [0, 8, 0]
    assert p["seg_kv_end"].tolist() == [8, 10, 4]
    assert p["seg_partial"].tolist() == [0, 1, -1]
    assert p["tile_first_partial"].tolist() == [0, -1]
    assert p["tile_num_partials"].tolist() == [2, 0]
    assert p["merge_list"].tolist() == [0]


def test_append_causal_hand_example():
    # one request, 20 keys (2 pages of 16, 4 valid in the last), 5 queries, 2 kv heads,
    # tile_q 2, tile_kv 8, causal. Query tiles see 15+2=17, 15+4=19, 15+5=20 keys ->
    # 3 blocks each; 6 tiles (h0: qt0..2, h1: qt0..2) = 18 blocks; W 4 -> quota 5.
    p = plan_ref(KIND_APPEND, 1, [0, 2], [4], 16, 2, 4, 8, qo_indptr=[0, 5], tile_q=2, causal=True)
    assert p["tile_h"].tolist() == [0, 0, 0, 1, 1, 1]
    assert p["tile_qt"].tolist() == [0, 1, 2, 0, 1, 2]
    assert p["worker_seg_indptr"].tolist() == [0, 2, 5, 7, 8]
    assert p["seg_tile"].tolist() == [0, 1, 1, 2, 3, 3, 4, 5]
    assert p["seg_kv_begin"].tolist() == [0, 0, 16, 0, 0, 8, 0, 0]
    assert p["seg_kv_end"].tolist() == [17, 16, 19, 20, 8, 17, 19, 20]
    assert p["seg_partial"].tolist() == [-1, 0, 1, -1, 2, 3, -1, -1]
    assert p["merge_list"].tolist() == [1, 3]
    assert p["tile_first_partial"].tolist() == [-1, 0, -1, 2, -1, -1]


def test_decode_head_groups_hand_example():
    # 2 requests of 10 and 4 keys, 4 kv heads in groups of 2, tile_kv 4, W 3.
    # Tiles (b, h): (0, 0) (0, 2) cost 3 blocks each, (1, 0) (1, 2) cost 1: N = 8,
    # quota 3. Worker 0: tile 0 whole. Worker 1: tile 1 whole. Worker 2: tiles 2, 3.
    p = plan_ref(KIND_DECODE, 2, [0, 3, 4], [2, 4], 4, 4, 3, 4, heads_per_tile=2)
    assert p["tile_b"].tolist() == [0, 0, 1, 1]
    assert p["tile_h"].tolist() == [0, 2, 0, 2]
    assert p["quota"].tolist() == [3]
    assert p["worker_seg_indptr"].tolist() == [0, 1, 2, 4]
    assert p["seg_kv_end"].tolist() == [10, 10, 4, 4]
    assert p["seg_partial"].tolist() == [-1, -1, -1, -1]
    assert p["merge_list"].tolist() == []
    with pytest.raises(PlanError):
        plan_ref(KIND_DECODE, 2, [0, 3, 4], [2, 4], 4, 4, 3, 4, heads_per_tile=3)


def test_empty_request_still_gets_a_block():
    p = plan_ref(KIND_DECODE, 3, [0, 0, 2, 2], [0, 3, 0], 4, 1, 8, 64)
    assert p["num_blocks"].tolist() == [3]
    assert p["seg_kv_begin"].tolist() == [0, 0, 0]
    assert p["seg_kv_end"].tolist() == [0, 7, 0]


@pytest.mark.parametrize("args", [
    dict(kv_indptr=[0, 2, 1], lpl=[1, 1]),      # decreasing indptr
    dict(kv_indptr=[1, 2, 3], lpl=[1, 1]),      # indptr not starting at 0
    dict(kv_indptr=[0, 1, 2], lpl=[0, 1]),      # last_page_len 0 with pages
    dict(kv_indptr=[0, 1, 2], lpl=[1, 5]),      # last_page_len > page size
])
def test_validation(args):
    with pytest.raises(PlanError):
        plan_ref(KIND_DECODE, 2, args["kv_indptr"], args["lpl"], 4, 1, 4, 16)


def test_causal_needs_qo_not_above_kv():
    with pytest.raises(PlanError):
        plan_ref(KIND_APPEND, 1, [0, 1], [3], 4, 1, 4, 16, qo_indptr=[0, 4], tile_q=2, causal=True)
    plan_ref(KIND_APPEND, 1, [0, 1], [3], 4, 1, 4, 16, qo_indptr=[0, 4], tile_q=2, causal=False)


def check_invariants(p, W, Tk, extents, contiguous=True):
    """contiguous: a tile's segments are adjacent in the listing (plain
    Stream-K); co-scheduled plans list them worker by worker."""
    T = len(extents)
    S = len(p["seg_tile"])
    quota = int(p["quota"][0])
    ind = p["worker_seg_indptr"]
    assert ind[0] == 0 and ind[-1] == S and np.all(np.diff(ind) >= 0)
    assert S <= T + W - 1
    # exact cover of every tile's blocks, in kv order
    for t in range(T):
        segs = np.nonzero(p["seg_tile"] == t)[0]
        assert len(segs) >= 1
        if contiguous:
            assert np.all(np.diff(segs) == 1)
        b = p["seg_kv_begin"][segs]
        e = p["seg_kv_end"][segs]
        assert b[0] == 0 and e[-1] == extents[t]
        assert np.all(b[1:] == e[:-1]) and np.all(b % Tk == 0)
        if len(segs) == 1:
            assert p["seg_partial"][segs[0]] == -1 and p["tile_first_partial"][t] == -1
        else:
            slots = p["seg_partial"][segs]
            assert np.all(np.diff(slots) == 1) and slots[0] == p["tile_first_partial"][t]
            assert p["tile_num_partials"][t] == len(segs)
    # split tiles take consecutive slot runs in tile order
    firsts = [int(p["tile_first_partial"][t]) for t in range(T) if p["tile_num_partials"][t] > 1]
    assert firsts == sorted(firsts)
    # worker loads stay within the quota
    for w in range(W):
        blocks = 0
        for s in range(ind[w], ind[w + 1]):
            blocks += max(1, -(-(int(p["seg_kv_end"][s]) - int(p["seg_kv_begin"][s])) // Tk))
        assert blocks <= quota
    used = p["seg_partial"][p["seg_partial"] >= 0]
    assert np.array_equal(np.sort(used), np.arange(len(used)))
    assert p["merge_list"].tolist() == [t for t in range(T) if p["tile_num_partials"][t] > 1]


@settings(max_examples=150, deadline=None)
@given(st.data())
def test_invariants_random(data):
    B = data.draw(st.integers(0, 9))
    P = data.draw(st.sampled_from([1, 3, 16, 256]))
    Hkv = data.draw(st.integers(1, 4))
    hpt = data.draw(st.sampled_from([d for d in (1, 2, 4) if Hkv % d == 0]))
    W = data.draw(st.integers(1, 40) | st.sampled_from([64, 96, 128]))
    Tk = data.draw(st.sampled_from([1, 16, 64]))
    kv_len = data.draw(st.lists(st.integers(0, 700), min_size=B, max_size=B))
    npg = [-(-n // P) for n in kv_len]
    indptr = np.concatenate([[0], np.cumsum(npg)]).astype(int)
    lpl = [n - (k - 1) * P if k else 0 for n, k in zip(kv_len, npg)]
    append = data.draw(st.booleans())
    if not append:
        p = plan_ref(KIND_DECODE, B, indptr, lpl, P, Hkv, W, Tk, heads_per_tile=hpt)
        ext = [n for n in kv_len for _ in range(Hkv // hpt)]
    else:
        causal = data.draw(st.booleans())
        Tq = data.draw(st.sampled_from([1, 4, 32]))
        qo = [data.draw(st.integers(0, n if causal else 90)) for n in kv_len]
        qo_indptr = np.concatenate([[0], np.cumsum(qo)]).astype(int)
        p = plan_ref(KIND_APPEND, B, indptr, lpl, P, Hkv, W, Tk, qo_indptr=qo_indptr,
                     tile_q=Tq, causal=causal, heads_per_tile=hpt)
        ext = []
        for n, m in zip(kv_len, qo):
            for _ in range(Hkv // hpt):
                for qt in range(-(-m // Tq)):
                    ext.append(n - m + min((qt + 1) * Tq, m) if causal else n)
    check_invariants(p, W, Tk, ext, contiguous=co_lanes(KIND_APPEND if append else KIND_DECODE, W) == 1)


def test_co_scheduled_append_hand_example():
    # The causal append example above on W = 16 workers: 2 per XCD, so units of
    # K = 2 tiles. Head 0's tiles 0, 1 form unit 0 and tile 2 is queued; head
    # 1's tiles 3, 4 form unit 1, and its tile 5 completes the queued unit 2
    # (2, 5). Unit 1 is odd, so its slots go to the lanes in reverse: lane 0
    # runs tiles 0, 4, 2 and lane 1 tiles 1, 3, 5. Units cost 3 blocks each:
    # 9 blocks over 8 groups -> quota 2. Group 0 (workers 0, 1): unit 0 blocks
    # 0-1. Group 1 (workers 2, 3): unit 0 block 2, unit 1 block 0. Group 2:
    # unit 1 blocks 1-2. Group 3: unit 2 blocks 0-1; group 4: its block 2.
    # Every tile is cut in two; slots run in tile order (tile t takes 2t, 2t + 1).
    p = plan_ref(KIND_APPEND, 1, [0, 2], [4], 16, 2, 16, 8, qo_indptr=[0, 5], tile_q=2,
                 causal=True)
    assert co_lanes(KIND_APPEND, 16) == 2
    assert p["quota"].tolist() == [2]
    assert p["worker_seg_indptr"].tolist() == [0, 1, 2, 4, 6, 7, 8, 9, 10, 11, 12] + [12] * 6
    assert p["seg_tile"].tolist() == [0, 1, 0, 4, 1, 3, 4, 3, 2, 5, 2, 5]
    assert p["seg_kv_begin"].tolist() == [0, 0, 16, 0, 16, 0, 8, 8, 0, 0, 16, 16]
    assert p["seg_kv_end"].tolist() == [16, 16, 17, 8, 19, 8, 19, 17, 16, 16, 20, 20]
    assert p["seg_partial"].tolist() == [0, 2, 1, 8, 3, 6, 9, 7, 4, 10, 5, 11]
    assert p["tile_first_partial"].tolist() == [0, 2, 4, 6, 8, 10]
    assert p["merge_list"].tolist() == [0, 1, 2, 3, 4, 5]
    # the same plan without co-scheduling is the plain Stream-K split
    q = plan_ref(KIND_APPEND, 1, [0, 2], [4], 16, 2, 16, 8, qo_indptr=[0, 5], tile_q=2,
                 causal=True, lanes=1)
    assert q["quota"].tolist() == [2]
    assert q["seg_tile"].tolist() == [0, 0, 1, 1, 2, 2, 3, 3, 4, 4, 5, 5]


def test_co_lanes_rule():
    assert [co_lanes(KIND_APPEND, w) for w in (8, 16, 24, 32, 48, 64, 96, 224, 256, 512)] == \
        [1, 2, 1, 4, 2, 8, 4, 4, 8, 8]
    assert co_lanes(KIND_APPEND, 20) == 1 and co_lanes(KIND_DECODE, 256) == 1
    assert co_lanes(KIND_APPEND, 256, no_split=True) == 1


@settings(max_examples=60, deadline=None)
@given(st.data())
def test_co_scheduled_lanes_share_keys(data):
    """Non-causal requests whose query tiles come in whole units: the K workers
    of each group (within one XCD's block of workers) walk the same key ranges,
    segment by segment, of tiles of one (request, kv head), and the plan
    covers every tile exactly once."""
    W = data.draw(st.sampled_from([16, 32, 64, 128, 256]))
    K = co_lanes(KIND_APPEND, W)
    assert K > 1 and (W // 8) % K == 0
    B = data.draw(st.integers(1, 6))
    Hkv = data.draw(st.integers(1, 3))
    Tq = data.draw(st.sampled_from([4, 32]))
    kv_len = data.draw(st.lists(st.integers(1, 900), min_size=B, max_size=B))
    qo = [K * Tq * data.draw(st.integers(0, 3)) for _ in kv_len]
    indptr = np.concatenate([[0], np.cumsum([-(-n // 16) for n in kv_len])]).astype(int)
    lpl = [n - (-(-n // 16) - 1) * 16 for n in kv_len]
    qo_indptr = np.concatenate([[0], np.cumsum(qo)]).astype(int)
    p = plan_ref(KIND_APPEND, B, indptr, lpl, 16, Hkv, W, 64, qo_indptr=qo_indptr, tile_q=Tq,
                 causal=False)
    ind = p["worker_seg_indptr"]
    for g in range(W // K):
        lanes = [range(ind[g * K + j], ind[g * K + j + 1]) for j in range(K)]
        assert len({len(r) for r in lanes}) == 1
        for segs in zip(*lanes):
            t = [int(p["seg_tile"][i]) for i in segs]
            assert len({(int(p["tile_b"][x]), int(p["tile_h"][x])) for x in t}) == 1
            assert len({int(p["tile_qt"][x]) for x in t}) == K
            assert len({(int(p["seg_kv_begin"][i]), int(p["seg_kv_end"][i])) for i in segs}) == 1
    ext = [n for n, m in zip(kv_len, qo) for _ in range(Hkv) for _ in range(m // Tq)]
    check_invariants(p, W, 64, ext, contiguous=False)


def test_no_split_hand_example():
    # The decode example above without load balancing: worker t takes tile t
    # whole. Tile 0 (10 keys, 3 blocks) is one segment [0, 10) on worker 0,
    # tile 1 (4 keys) one segment [0, 4) on worker 1; worker 2 gets nothing;
    # no partial states and nothing to merge.
    p = plan_ref(KIND_DECODE, 2, [0, 3, 4], [2, 4], 4, 1, 3, 4, no_split=True)
    assert p["worker_seg_indptr"].tolist() == [0, 1, 2, 2]
    assert p["seg_tile"].tolist() == [0, 1]
    assert p["seg_kv_begin"].tolist() == [0, 0]
    assert p["seg_kv_end"].tolist() == [10, 4]
    assert p["seg_partial"].tolist() == [-1, -1]
    assert p["num_partials"].tolist() == [0]
    assert p["merge_list"].tolist() == []
    with pytest.raises(PlanError):
        plan_ref(KIND_DECODE, 2, [0, 3, 4], [2, 4], 4, 1, 1, 4, no_split=True)


def test_no_split_covers_each_tile_once_on_its_own_worker():
    rng = np.random.Generator(np.random.PCG64(77))
    kv = rng.integers(0, 500, size=9)
    npg = -(-kv // 16)
    indptr = np.concatenate([[0], np.cumsum(npg)])
    lpl = np.where(npg > 0, kv - (npg - 1) * 16, 0)
    p = plan_ref(KIND_DECODE, 9, indptr, lpl, 16, 8, 20, 64, heads_per_tile=4, no_split=True)
    T = len(p["tile_b"])
    assert T == 18
    wsi = p["worker_seg_indptr"]
    assert (np.diff(wsi)[:T] == 1).all() and (np.diff(wsi)[T:] == 0).all()
    assert p["seg_tile"].tolist() == list(range(T))
    assert (p["seg_kv_begin"] == 0).all()
    assert p["seg_kv_end"].tolist() == [int(kv[b]) for b in p["tile_b"]]
