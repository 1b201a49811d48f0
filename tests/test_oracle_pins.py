"""Pins of the fp64 oracle to facts outside itself (CPU only).

Each test checks the oracle against something it does not compute the same way:
exact constants of the storage formats, closed forms of the softmax, invariants
that the pages' claims imply, and a library routine (PyTorch's scaled-dot-product
attention in float64) on tiny inputs. A plausible slip in the oracle (a dropped
term, a wrong sign, index or page, a transposed operand) fails at least one.
"""
import math

import numpy as np
import pytest

from oracle import attention as ora
from attention_bsr_paged_amd import workloads as wl


def rnd(seed, *shape):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape)


# ----------------------------------------------------------------------------
# storage formats: exact constants from the IEEE binary16 / bfloat16 definitions
# ----------------------------------------------------------------------------
def test_storage_constants():
    bf = np.array([0x3F80, 0xC000, 0x0001, 0x7F7F, 0x3EAA], dtype=np.uint16)
    got = ora.storage_to_f64(bf, "bf16")
    assert got[0] == 1.0 and got[1] == -2.0
    assert got[2] == 2.0 ** -133                       # smallest bf16 subnormal
    assert got[3] == (2 - 2.0 ** -7) * 2.0 ** 127      # largest finite bf16
    assert got[4] == 0.33203125                        # 0x3EAA = 1.328125 * 2^-2
    fp = np.array([0x3C00, 0x0001, 0x7BFF, 0xB800], dtype=np.uint16)
    got = ora.storage_to_f64(fp, "fp16")
    assert list(got) == [1.0, 2.0 ** -24, 65504.0, -0.5]


def test_generator_rounding_is_rne():
    # 1 + 2^-8 is a bf16 tie: it rounds to the even neighbour 1.0; 1 + 3*2^-8 rounds up
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -9], dtype=np.float32)
    got = ora.storage_to_f64(wl.round_to_bf16_bits(x), "bf16")
    assert list(got) == [1.0, 1 + 2 ** -6, -1.0]


# ----------------------------------------------------------------------------
# page table walk
# ----------------------------------------------------------------------------
def test_walk_pages_hand_example():
    # pool of 4 pages of 4 slots; slot value = 10 * page + slot
    P = 4
    pool = (10 * np.arange(4)[:, None] + np.arange(P)[None, :]).astype(np.float64)[:, :, None, None]
    indptr = np.array([0, 3, 3, 4])
    indices = np.array([2, 0, 3, 1])
    lpl = np.array([2, 0, 4])
    rows0 = ora.walk_pages(pool, indptr, indices, lpl, P, 0)[:, 0, 0]
    assert list(rows0) == [20, 21, 22, 23, 0, 1, 2, 3, 30, 31]
    assert ora.walk_pages(pool, indptr, indices, lpl, P, 1).shape[0] == 0
    assert list(ora.walk_pages(pool, indptr, indices, lpl, P, 2)[:, 0, 0]) == [10, 11, 12, 13]
    assert [ora.request_kv_len(indptr, lpl, P, b) for b in range(3)] == [10, 0, 4]


# ----------------------------------------------------------------------------
# attention: closed forms
# ----------------------------------------------------------------------------
def test_zero_query_gives_mean_and_log_count():
    K, V = rnd(1, 37, 16), rnd(2, 37, 16)
    o, lse = ora.attend(np.zeros((3, 16)), K, V, 0.25, visible=[37, 5, 1])
    assert np.allclose(o[0], V.mean(0), atol=1e-14)
    assert np.allclose(o[1], V[:5].mean(0), atol=1e-14)
    assert np.allclose(o[2], V[0], atol=1e-15)
    assert np.allclose(lse, [math.log(37), math.log(5), 0.0], atol=1e-14)


def test_constant_values_and_single_key():
    q, K = rnd(3, 2, 8), rnd(4, 9, 8)
    V = np.tile(np.arange(8.0), (9, 1))
    o, _ = ora.attend(q, K, V, 0.7)
    assert np.allclose(o, np.arange(8.0), atol=1e-13)
    o1, l1 = ora.attend(q, K[:1], rnd(5, 1, 8), 0.7)
    assert np.allclose(o1, rnd(5, 1, 8), atol=1e-15)
    assert np.allclose(l1, 0.7 * (q @ K[0]), atol=1e-14)


def test_two_equal_logits_give_log2():
    q = np.array([[1.0, 0.0]])
    K = np.array([[2.0, 5.0], [2.0, -3.0]])   # both logits = 2 * scale
    V = np.array([[1.0, 0.0], [0.0, 1.0]])
    o, lse = ora.attend(q, K, V, 0.5)
    assert np.allclose(o, [[0.5, 0.5]], atol=1e-15)
    assert abs(lse[0] - (1.0 + math.log(2))) < 1e-15


def test_one_hot_key_selects_its_value():
    # key 11 is a large multiple of q: its weight dominates every other key
    d, n = 32, 40
    q = rnd(6, 1, d)
    K = rnd(7, n, d)
    K[11] = 60.0 * q[0] / np.linalg.norm(q[0])
    V = rnd(8, n, d)
    o, _ = ora.attend(q, K, V, 1.0 / math.sqrt(d))
    assert np.allclose(o[0], V[11], atol=1e-12)


def test_empty_visible_set():
    o, lse = ora.attend(rnd(9, 2, 4), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))
    o, lse = ora.attend(rnd(9, 2, 4), rnd(10, 3, 4), rnd(11, 3, 4), 1.0, visible=[0, 3])
    assert np.all(o[0] == 0) and np.isneginf(lse[0]) and np.isfinite(lse[1])


# ----------------------------------------------------------------------------
# attention: a library routine on tiny inputs (torch SDPA in float64 on the CPU)
# ----------------------------------------------------------------------------
def _sdpa(Q, K, V, scale, mask=None):
    import torch
    import torch.nn.functional as F
    q = torch.from_numpy(Q)[None]      # [1, r, d] (one "head")
    k = torch.from_numpy(K)[None]
    v = torch.from_numpy(V)[None]
    m = None if mask is None else torch.from_numpy(mask)[None]
    return F.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)[0].numpy()


@pytest.mark.parametrize("P", [1, 3, 16])
def test_paged_decode_matches_sdpa(P):
    w = wl.small_decode(21 + P, [0, 1, 17, 40], P, num_qo_heads=4, num_kv_heads=2, head_dim=8,
                        dtype="bf16")
    kv = w.kv
    o, lse = ora.decode_workload(w)
    for b in range(w.batch):
        n = int(kv.kv_len[b])
        if n == 0:
            assert np.all(o[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        # assemble K, V from the page table independently (flat token -> page/slot)
        tok = np.arange(n)
        pages = kv.kv_indices[kv.kv_indptr[b] + tok // P]
        K = ora.storage_to_f64(kv.k_pages[pages, tok % P], "bf16")
        V = ora.storage_to_f64(kv.v_pages[pages, tok % P], "bf16")
        q = ora.storage_to_f64(w.q[b], "bf16")
        for hq in range(4):
            ref = _sdpa(q[hq:hq + 1], K[:, hq // 2], V[:, hq // 2], w.sm_scale)
            assert np.allclose(o[b, hq], ref[0], atol=1e-12)


def test_causal_append_matches_sdpa_bottom_right():
    w = wl.small_append(31, [1, 5, 7], [9, 5, 20], 4, num_qo_heads=2, num_kv_heads=1,
                        head_dim=8, dtype="fp16", causal=True)
    o, _ = ora.append_workload(w)
    kv = w.kv
    for b in range(3):
        q0, q1 = w.qo_indptr[b], w.qo_indptr[b + 1]
        n, m = int(kv.kv_len[b]), int(q1 - q0)
        tok = np.arange(n)
        pages = kv.kv_indices[kv.kv_indptr[b] + tok // 4]
        K = ora.storage_to_f64(kv.k_pages[pages, tok % 4, 0], "fp16")
        V = ora.storage_to_f64(kv.v_pages[pages, tok % 4, 0], "fp16")
        # bottom-right aligned causal mask: query i sees keys j <= i + (n - m)
        mask = np.tril(np.ones((m, n), dtype=bool), k=n - m)
        for hq in range(2):
            Q = ora.storage_to_f64(w.q[q0:q1, hq], "fp16")
            ref = _sdpa(Q, K, V, w.sm_scale, mask)
            assert np.allclose(o[q0:q1, hq], ref, atol=1e-12)


# ----------------------------------------------------------------------------
# attention: invariants the pages' claims imply
# ----------------------------------------------------------------------------
def test_contiguous_equals_single_page_and_page_size_independence():
    # one logical KV in page sizes 1, 3, 16 and one page of size kv_len
    rng = np.random.Generator(np.random.PCG64(41))
    n, Hkv, d = 45, 2, 16
    Kt = wl.normal_bits(rng, (n, Hkv, d), "bf16")
    Vt = wl.normal_bits(rng, (n, Hkv, d), "bf16")
    q = wl.normal_bits(rng, (1, 4, d), "bf16")
    res = []
    for P in (1, 3, 16, n):
        npg = -(-n // P)
        perm = rng.permutation(npg + 2)
        kp = np.zeros((npg + 2, P, Hkv, d), np.uint16)
        vp = np.zeros_like(kp)
        for i in range(npg):
            seg = slice(i * P, min(n, (i + 1) * P))
            kp[perm[i], : seg.stop - seg.start] = Kt[seg]
            vp[perm[i], : seg.stop - seg.start] = Vt[seg]
        indptr = np.array([0, npg])
        lpl = np.array([n - (npg - 1) * P])
        res.append(ora.paged_decode(q, kp, vp, indptr, perm[:npg], lpl, P, "bf16", Hkv))
    for o, l in res[1:]:
        assert np.allclose(o, res[0][0], atol=1e-13) and np.allclose(l, res[0][1], atol=1e-13)


def test_page_permutation_invariance():
    w = wl.small_decode(51, [33, 70], 8, 4, 2, head_dim=16, extra_pages=5)
    kv = w.kv
    o, l = ora.decode_workload(w)
    perm = np.random.Generator(np.random.PCG64(52)).permutation(kv.num_pages)
    kp = np.empty_like(kv.k_pages)
    vp = np.empty_like(kv.v_pages)
    kp[perm] = kv.k_pages
    vp[perm] = kv.v_pages
    o2, l2 = ora.paged_decode(w.q, kp, vp, kv.kv_indptr, perm[kv.kv_indices], kv.kv_last_page_len,
                              8, "bf16", 2)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def test_wrong_page_changes_lse():
    # swapping two logical pages inside a request is invisible (a permutation of keys),
    # but pointing a slot at an unused page must move lse
    w = wl.small_decode(53, [64], 16, 4, 2, head_dim=16, extra_pages=2)
    kv = w.kv
    _, l = ora.decode_workload(w)
    idx = kv.kv_indices.copy()
    idx[[0, 1]] = idx[[1, 0]]
    _, l_sw = ora.paged_decode(w.q, kv.k_pages, kv.v_pages, kv.kv_indptr, idx, kv.kv_last_page_len,
                               16, "bf16", 2)
    assert np.allclose(l, l_sw, atol=1e-13)
    unused = sorted(set(range(kv.num_pages)) - set(kv.kv_indices.tolist()))[0]
    idx = kv.kv_indices.copy()
    idx[2] = unused
    _, l_bad = ora.paged_decode(w.q, kv.k_pages, kv.v_pages, kv.kv_indptr, idx,
                                kv.kv_last_page_len, 16, "bf16", 2)
    assert np.max(np.abs(l - l_bad)) > 1e-3


@pytest.mark.parametrize("cuts", [[1], [7, 30], [5, 6, 44]])
def test_merge_of_splits_equals_unsplit(cuts):
    q, K, V = rnd(61, 5, 16), rnd(62, 45, 16), rnd(63, 45, 16)
    full = ora.attend(q, K, V, 0.3)
    edges = [0] + cuts + [45]
    parts = [ora.attend(q, K[a:b], V[a:b], 0.3) for a, b in zip(edges[:-1], edges[1:])]
    o, lse = ora.merge(parts)
    assert np.allclose(o, full[0], atol=1e-13) and np.allclose(lse, full[1], atol=1e-13)
    # order of the parts does not matter
    o2, l2 = ora.merge(parts[::-1])
    assert np.allclose(o2, o, atol=1e-14) and np.allclose(l2, lse, atol=1e-14)


def test_merge_closed_forms():
    oa, ob = rnd(64, 3, 4), rnd(65, 3, 4)
    la = np.array([0.5, -np.inf, -np.inf])
    lb = np.array([0.5, 2.0, -np.inf])
    o, lse = ora.merge([(oa, la), (ob, lb)])
    assert np.allclose(o[0], (oa[0] + ob[0]) / 2) and abs(lse[0] - (0.5 + math.log(2))) < 1e-15
    assert np.allclose(o[1], ob[1]) and lse[1] == 2.0
    assert np.all(o[2] == 0) and np.isneginf(lse[2])
    # weights follow exp(lse_i - lse): lse_a = ln 3, lse_b = ln 1 -> 3/4, 1/4
    o, lse = ora.merge([(oa[:1], np.array([math.log(3)])), (ob[:1], np.array([0.0]))])
    assert np.allclose(o[0], 0.75 * oa[0] + 0.25 * ob[0], atol=1e-15)
    assert abs(lse[0] - math.log(4)) < 1e-15


def test_gqa_equals_mha_with_repeated_heads():
    w = wl.small_decode(71, [29, 50], 4, 8, 2, head_dim=16)
    kv = w.kv
    o, l = ora.decode_workload(w)
    rep = lambda p: np.repeat(p, 4, axis=2)     # kv head h -> qo heads 4h..4h+3
    o2, l2 = ora.paged_decode(w.q, rep(kv.k_pages), rep(kv.v_pages), kv.kv_indptr, kv.kv_indices,
                              kv.kv_last_page_len, 4, "bf16", 8)
    assert np.allclose(o, o2, atol=1e-13) and np.allclose(l, l2, atol=1e-13)


def test_causal_row_equals_decode_over_prefix():
    w = wl.small_append(81, [6], [19], 4, 4, 2, head_dim=16, causal=True)
    kv = w.kv
    o, l = ora.append_workload(w)
    for i in range(6):
        # query i sees the first 19 - 6 + i + 1 keys: a decode over a truncated table
        n = 19 - 6 + i + 1
        npg = -(-n // 4)
        od, ld = ora.paged_decode(w.q[i:i + 1], kv.k_pages, kv.v_pages, np.array([0, npg]),
                                  kv.kv_indices[:npg], np.array([n - (npg - 1) * 4]), 4, "bf16", 2)
        assert np.allclose(o[i], od[0], atol=1e-13) and np.allclose(l[i], ld[0], atol=1e-13)


def test_non_causal_append_rows_are_decodes():
    w = wl.small_append(82, [3, 4], [10, 2], 4, 4, 2, head_dim=16, causal=False)
    kv = w.kv
    o, l = ora.append_workload(w)
    for b in range(2):
        for j in range(w.qo_indptr[b], w.qo_indptr[b + 1]):
            s = slice(kv.kv_indptr[b], kv.kv_indptr[b + 1])
            od, ld = ora.paged_decode(w.q[j:j + 1], kv.k_pages, kv.v_pages,
                                      np.array([0, s.stop - s.start]), kv.kv_indices[s],
                                      kv.kv_last_page_len[b:b + 1], 4, "bf16", 2)
            assert np.allclose(o[j], od[0], atol=1e-13) and np.allclose(l[j], ld[0], atol=1e-13)


# ----------------------------------------------------------------------------
# RoPE
# ----------------------------------------------------------------------------
def test_rope_closed_forms():
    d, theta = 128, 500000.0
    e = np.eye(d)
    p = 7.0
    r0 = ora.rope_rotate(e[0], p, theta)             # pair 0 turns by angle p
    assert np.allclose(r0[[0, 64]], [math.cos(p), math.sin(p)], atol=1e-15)
    assert np.allclose(np.delete(r0, [0, 64]), 0)
    r64 = ora.rope_rotate(e[64], p, theta)
    assert np.allclose(r64[[0, 64]], [-math.sin(p), math.cos(p)], atol=1e-15)
    a1 = p * theta ** (-2.0 / d)                     # pair 1 turns by p * theta^(-2/d)
    r1 = ora.rope_rotate(e[1], p, theta)
    assert np.allclose(r1[[1, 65]], [math.cos(a1), math.sin(a1)], atol=1e-15)
    a63 = p * theta ** (-126.0 / d)
    r127 = ora.rope_rotate(e[127], p, theta)
    assert np.allclose(r127[[63, 127]], [-math.sin(a63), math.cos(a63)], atol=1e-15)


def test_rope_complex_form_and_invariants():
    d, theta = 128, 500000.0
    x = rnd(91, 6, d)
    pos = np.array([0, 1, 17, 8191, 9000, 40000])
    got = ora.rope_rotate(x, pos, theta)
    # complex form: z_j = x_j + i x_{j+d/2} is multiplied by exp(i pos theta^(-2j/d))
    z = (x[:, :64] + 1j * x[:, 64:]) * np.exp(1j * np.outer(pos, theta ** (-np.arange(64) * 2.0 / d)))
    assert np.allclose(got, np.concatenate([z.real, z.imag], axis=1), atol=1e-12)
    assert np.allclose(got[0], x[0], atol=0)                          # position 0: identity
    assert np.allclose(np.linalg.norm(got, axis=1), np.linalg.norm(x, axis=1), atol=1e-12)
    # logits depend only on the position difference
    q, k = rnd(92, d), rnd(93, d)
    s1 = ora.rope_rotate(q, 9000, theta) @ ora.rope_rotate(k, 8000, theta)
    s2 = ora.rope_rotate(q, 1234, theta) @ ora.rope_rotate(k, 234, theta)
    assert abs(s1 - s2) < 1e-10


# ----------------------------------------------------------------------------
# cascade: equals flat attention over prefix || suffix
# ----------------------------------------------------------------------------
def test_cascade_equals_flat():
    rng = np.random.Generator(np.random.PCG64(101))
    B, Hq, Hkv, d, pre_len = 3, 4, 2, 16, 40
    prefix = wl.make_paged_kv(rng, np.array([pre_len]), 16, Hkv, d, "bf16", extra_pages=1)
    suf = np.array([5, 17, 1])
    kv = wl.make_paged_kv(rng, suf, 4, Hkv, d, "bf16", extra_pages=2)
    q = wl.normal_bits(rng, (B, Hq, d), "bf16")
    for theta in (0.0, 500000.0):
        o, l = ora.cascade_decode(q, prefix.k_pages, prefix.v_pages, prefix.kv_indptr,
                                  prefix.kv_indices, prefix.kv_last_page_len, 16, kv.k_pages,
                                  kv.v_pages, kv.kv_indptr, kv.kv_indices, kv.kv_last_page_len, 4,
                                  "bf16", Hkv, rope_theta=theta)
        for b in range(B):
            Kp = ora.walk_pages(prefix.k_pages, prefix.kv_indptr, prefix.kv_indices,
                                prefix.kv_last_page_len, 16, 0)
            Vp = ora.walk_pages(prefix.v_pages, prefix.kv_indptr, prefix.kv_indices,
                                prefix.kv_last_page_len, 16, 0)
            Ks = ora.walk_pages(kv.k_pages, kv.kv_indptr, kv.kv_indices, kv.kv_last_page_len, 4, b)
            Vs = ora.walk_pages(kv.v_pages, kv.kv_indptr, kv.kv_indices, kv.kv_last_page_len, 4, b)
            # a single flat request holding prefix || suffix, pages of 1 token
            K = np.concatenate([Kp, Ks])[:, None]
            V = np.concatenate([Vp, Vs])[:, None]
            n = K.shape[0]
            of, lf = ora.paged_decode(q[b:b + 1], K, V, np.array([0, n]), np.arange(n),
                                      np.array([1]), 1, "bf16", Hkv, rope_theta=theta)
            assert np.allclose(o[b], of[0], atol=1e-13) and np.allclose(l[b], lf[0], atol=1e-13)


def test_page_example_shapes():
    """The pages' single-decode example: q [32,128], k/v [2048,32,128] fp16 -> o [32,128].

    A contiguous cache is one BSR page of size kv_len; it must equal the same
    keys stored in 128 pages of 16 in shuffled physical order.
    """
    import json, os
    ex = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "single_decode_example.json")))
    rng = np.random.Generator(np.random.PCG64(5))
    n, Hkv, d = ex["k_shape"]
    q = wl.normal_bits(rng, (1,) + tuple(ex["q_shape"]), ex["dtype"])
    k = wl.normal_bits(rng, (1, n, Hkv, d), ex["dtype"])
    v = wl.normal_bits(rng, (1, n, Hkv, d), ex["dtype"])
    o, l = ora.paged_decode(q, k, v, [0, 1], [0], [n], n, ex["dtype"], Hkv)
    assert list(o[0].shape) == ex["output_shape"]
    perm = rng.permutation(n // 16)
    kp = np.empty((n // 16, 16, Hkv, d), np.uint16)
    vp = np.empty_like(kp)
    kp[perm] = k[0].reshape(n // 16, 16, Hkv, d)
    vp[perm] = v[0].reshape(n // 16, 16, Hkv, d)
    o2, l2 = ora.paged_decode(q, kp, vp, [0, n // 16], perm, [16], 16, ex["dtype"], Hkv)
    assert np.allclose(o, o2, atol=1e-13) and np.allclose(l, l2, atol=1e-13)
