"""Reference work-unit planner (pure Python, integers only).

TEST INFRASTRUCTURE: only ``tests/`` may use it. The library's own C++ planner
must reproduce every array returned here bit for bit.

The paper summary ("图谱动态｜学苑周刊 NO.266", section 动态负载均衡调度)
states the scheme only in words: attention is cut into work units that are
spread over the compute units to minimise imbalance, in the spirit of Stream-K;
a plan is made on the CPU from the length distribution and the GPU kernel, a
persistent kernel with a fixed grid and a preallocated workspace, follows it.
The concrete rule below is the plainest Stream-K reading of that passage:

1. Validate. kv_len_b = (n_b - 1) * page_size + last_page_len_b when request b
   owns n_b > 0 pages (last_page_len_b in [1, page_size]), else 0; indptr must
   be non-decreasing and start at 0; a causal append needs qo_len_b <= kv_len_b.
2. Tiles, in order: request b, then kv-head group, then query tile qt. A group
   is heads_per_tile consecutive kv heads starting at h (a property of the
   kernel that runs the plan: how many heads one worker covers at once; the
   pages leave it open). Decode has one tile per (b, group) (its rows are the
   qo heads of the group's kv heads). Append has ceil(qo_len_b / tile_q) query
   tiles per (b, group). A tile's extent is the number
   of keys its last row may see: kv_len_b - qo_len_b + min((qt + 1) * tile_q,
   qo_len_b) when causal, else kv_len_b. It costs nblk = max(1,
   ceil(extent / tile_kv)) blocks of tile_kv keys of all the group's heads (an
   empty tile still writes its (0, -inf)).
3. Partition. N = sum of nblk; quota = ceil(N / W); worker w owns the global
   block range [w * quota, min((w + 1) * quota, N)).
4. Segments are the intersections of a worker's range with one tile's blocks, in
   increasing global order: (tile, kv_begin, kv_end, worker), kv_begin =
   first local block * tile_kv, kv_end = min((last local block + 1) * tile_kv,
   extent).
5. A tile covered by one segment writes its output directly (partial = -1).
   Otherwise the tile enters the merge list, and the split tiles, in tile
   order, take consecutive runs of partial slots; a tile's segments fill its
   run in the order they are listed (kv order).
6. Co-scheduling (append plans with load balancing whose worker count W is a
   multiple of 8; the pages leave the order of the work units open, and this
   rule serves the kernels' placement of worker w on XCD w / (W / 8)): K = the
   largest of 8, 4, 2 dividing W / 8 (none: K = 1, steps 3-4 as written). K
   consecutive workers form a group; units of K tiles replace tiles and groups
   replace workers in steps 3-4. Walking the (request, kv-head group) runs of
   tiles in order, each run gives its whole K-tile units (consecutive query
   tiles) and queues its remaining tiles; every K queued tiles form a unit at
   that point, and a last incomplete one is padded with idle lanes. A unit
   costs the largest nblk of its tiles; quota = ceil(sum of unit costs / (W /
   K)); group g owns [g * quota, (g + 1) * quota) of unit blocks. Lane j of
   unit i is slot j when i is even and slot K - 1 - j when i is odd. Where
   group g meets unit i in its local blocks [lo, hi), lane j's tile t gets the
   segment [lo * tile_kv, min(min(hi, nblk_t) * tile_kv, extent_t)) on worker
   K g + j, unless lo >= nblk_t. Segments are listed worker by worker, each
   worker's in unit order; partial slots follow that listing (so each tile's
   slots are consecutive and in kv order).
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

KIND_DECODE = 0
KIND_APPEND = 1


class PlanError(ValueError):
    pass


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def kv_lengths(kv_indptr: Sequence[int], kv_last_page_len: Sequence[int], page_size: int,
               batch: int):
    if page_size < 1:
        raise PlanError("page_size must be >= 1")
    if len(kv_indptr) < batch + 1 or int(kv_indptr[0]) != 0:
        raise PlanError("kv_indptr must have batch+1 entries starting at 0")
    out = []
    for b in range(batch):
        n = int(kv_indptr[b + 1]) - int(kv_indptr[b])
        if n < 0:
            raise PlanError("kv_indptr must be non-decreasing")
        if n == 0:
            out.append(0)
            continue
        lpl = int(kv_last_page_len[b])
        if lpl < 1 or lpl > page_size:
            raise PlanError("kv_last_page_len must lie in [1, page_size]")
        out.append((n - 1) * page_size + lpl)
    return out


def co_lanes(kind: int, num_workers: int, no_split: bool = False) -> int:
    """Workers per co-scheduled group (rule 6 of the module docstring)."""
    if kind != KIND_APPEND or no_split or num_workers % 8:
        return 1
    for k in (8, 4, 2):
        if (num_workers // 8) % k == 0:
            return k
    return 1


def plan_ref(kind: int, batch: int, kv_indptr, kv_last_page_len, page_size: int,
             num_kv_heads: int, num_workers: int, tile_kv: int, qo_indptr=None,
             tile_q: int = 1, causal: bool = False,
             heads_per_tile: int = 1, no_split: bool = False,
             lanes: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Return the plan as int32 arrays (see the module docstring for the rule).

    ``no_split`` is the ablation without load balancing: worker t takes tile t
    whole (one segment, no partial states); ``num_workers`` must be at least
    the number of tiles, and the workers past them get nothing. ``lanes`` is
    the co-scheduling group size K (None: rule 6's choice; 1: plain Stream-K,
    as block-sparse plans use)."""
    if num_workers < 1 or tile_kv < 1 or tile_q < 1 or num_kv_heads < 1 or batch < 0:
        raise PlanError("bad sizes")
    if heads_per_tile < 1 or num_kv_heads % heads_per_tile:
        raise PlanError("heads_per_tile must divide num_kv_heads")
    kv_len = kv_lengths(kv_indptr, kv_last_page_len, page_size, batch)
    if kind == KIND_DECODE:
        qo_len = [1] * batch
        n_qt = [1] * batch
        causal = False
    else:
        if qo_indptr is None or int(qo_indptr[0]) != 0:
            raise PlanError("qo_indptr must start at 0")
        qo_len = []
        for b in range(batch):
            n = int(qo_indptr[b + 1]) - int(qo_indptr[b])
            if n < 0:
                raise PlanError("qo_indptr must be non-decreasing")
            if causal and n > kv_len[b]:
                raise PlanError("causal append needs qo_len <= kv_len")
            qo_len.append(n)
        n_qt = [_ceil_div(n, tile_q) for n in qo_len]

    tile_b, tile_h, tile_qt, extent, nblk = [], [], [], [], []
    for b in range(batch):
        for h in range(0, num_kv_heads, heads_per_tile):
            for qt in range(n_qt[b]):
                if causal:
                    e = kv_len[b] - qo_len[b] + min((qt + 1) * tile_q, qo_len[b])
                else:
                    e = kv_len[b]
                tile_b.append(b)
                tile_h.append(h)
                tile_qt.append(qt)
                extent.append(e)
                nblk.append(max(1, _ceil_div(e, tile_kv)))
    T = len(tile_b)
    N = sum(nblk)
    quota = _ceil_div(N, num_workers) if N else 1

    seg_tile, seg_begin, seg_end, seg_worker = [], [], [], []
    if no_split and T > num_workers:
        raise PlanError("one worker per tile needs num_workers >= the number of tiles")
    K = co_lanes(kind, num_workers, no_split) if lanes is None else int(lanes)
    if K > 1:
        if no_split or num_workers % K:
            raise PlanError("co-scheduling needs load balancing and K | num_workers")
        units, queued = [], []
        t0 = 0
        while t0 < T:
            t1 = t0 + 1
            while t1 < T and (tile_b[t1], tile_h[t1]) == (tile_b[t0], tile_h[t0]):
                t1 += 1
            whole = t0 + (t1 - t0) // K * K
            units += [list(range(i, i + K)) for i in range(t0, whole, K)]
            for i in range(whole, t1):
                queued.append(i)
                if len(queued) == K:
                    units.append(queued)
                    queued = []
            t0 = t1
        if queued:
            units.append(queued + [-1] * (K - len(queued)))
        cost = [max(nblk[t] for t in u if t >= 0) for u in units]
        quota = _ceil_div(sum(cost), num_workers // K) if units else 1
        per_worker = [[] for _ in range(num_workers)]
        g0 = 0
        for i, (u, c) in enumerate(zip(units, cost)):
            g1 = g0 + c
            grp = g0 // quota
            while grp * quota < g1:
                lo, hi = max(g0, grp * quota) - g0, min(g1, (grp + 1) * quota) - g0
                for j in range(K):
                    t = u[K - 1 - j] if i % 2 else u[j]
                    if t >= 0 and lo < nblk[t]:
                        per_worker[grp * K + j].append(
                            (t, lo * tile_kv, min(min(hi, nblk[t]) * tile_kv, extent[t])))
                grp += 1
            g0 = g1
        for w, lst in enumerate(per_worker):
            for t, kb, ke in lst:
                seg_tile.append(t)
                seg_begin.append(kb)
                seg_end.append(ke)
                seg_worker.append(w)
    g0 = 0
    for t in range(T if K == 1 else 0):
        if no_split:
            seg_tile.append(t)
            seg_begin.append(0)
            seg_end.append(extent[t])
            seg_worker.append(t)
            continue
        g1 = g0 + nblk[t]
        w = g0 // quota
        while w * quota < g1:
            lo = max(g0, w * quota)
            hi = min(g1, (w + 1) * quota)
            seg_tile.append(t)
            seg_begin.append((lo - g0) * tile_kv)
            seg_end.append(min((hi - g0) * tile_kv, extent[t]))
            seg_worker.append(w)
            w += 1
        g0 = g1
    S = len(seg_tile)

    nseg = [0] * T
    for t in seg_tile:
        nseg[t] += 1
    first_partial = [-1] * T
    num_partials = [0] * T
    slot = 0
    for t in range(T):
        if nseg[t] > 1:
            first_partial[t] = slot
            num_partials[t] = nseg[t]
            slot += nseg[t]
    seg_partial = []
    used = [0] * T
    for s in range(S):
        t = seg_tile[s]
        if nseg[t] == 1:
            seg_partial.append(-1)
        else:
            seg_partial.append(first_partial[t] + used[t])
            used[t] += 1
    merge_list = [t for t in range(T) if nseg[t] > 1]

    worker_seg_indptr = [0] * (num_workers + 1)
    for w in seg_worker:
        worker_seg_indptr[w + 1] += 1
    for w in range(num_workers):
        worker_seg_indptr[w + 1] += worker_seg_indptr[w]

    i32 = lambda x: np.asarray(x, dtype=np.int32)
    return {
        "num_blocks": i32([N]),
        "quota": i32([quota]),
        "num_partials": i32([slot]),
        "worker_seg_indptr": i32(worker_seg_indptr),
        "seg_tile": i32(seg_tile),
        "seg_kv_begin": i32(seg_begin),
        "seg_kv_end": i32(seg_end),
        "seg_partial": i32(seg_partial),
        "tile_b": i32(tile_b),
        "tile_h": i32(tile_h),
        "tile_qt": i32(tile_qt),
        "tile_first_partial": i32(first_partial),
        "tile_num_partials": i32(num_partials),
        "merge_list": i32(merge_list),
    }
