"""Pins of the oracle's block-sparse attention, page append and LLaMA 3.1 RoPE
scaling to facts outside themselves (CPU only).

- Hand-worked masks and page writes, written out element by element here.
- PyTorch's scaled-dot-product attention in float64 as a library special case.
- An explicit per-key loop with math.exp on tiny inputs.
- Closed forms and invariants: continuity of the scaled RoPE frequencies at the
  edges of the blended band, norm preservation.

A slip in the oracle fails at least one pin: swapped R and C, a transposed
block index, a wrong write position, or an inverted blend weight.
"""
import math

import numpy as np
import pytest

from oracle import attention as ora
from attention_bsr_paged_amd import workloads as wl


def _sdpa(Q, K, V, scale, mask=None):
    import torch
    import torch.nn.functional as F
    q = torch.from_numpy(Q)[None]
    k = torch.from_numpy(K)[None]
    v = torch.from_numpy(V)[None]
    m = None if mask is None else torch.from_numpy(mask)[None]
    return F.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)[0].numpy()


# ----------------------------------------------------------------------------
# block-sparse attention
# ----------------------------------------------------------------------------
def test_bsr_mask_hand_example():
    # M = 5 queries in row blocks of R = 2 (the last block has 1 query),
    # N = 6 keys in column blocks of C = 3: block row 0 sees column block 1,
    # block row 1 sees blocks 0 and 1, block row 2 sees nothing
    mask = ora.bsr_mask(5, 6, 2, 3, [0, 1, 3, 3], [1, 0, 1])
    want = np.array([
        [0, 0, 0, 1, 1, 1],
        [0, 0, 0, 1, 1, 1],
        [1, 1, 1, 1, 1, 1],
        [1, 1, 1, 1, 1, 1],
        [0, 0, 0, 0, 0, 0],
    ], dtype=bool)
    assert np.array_equal(mask, want)
    # unsorted column lists give the same mask
    assert np.array_equal(ora.bsr_mask(5, 6, 2, 3, [0, 1, 3, 3], [1, 1, 0]), want)


def test_bsr_attention_brute_force_loop():
    # explicit per-query, per-key loop with math.exp (no matrix products)
    w = wl.small_bsr(11, M=7, N=12, R=3, C=4, num_qo_heads=4, num_kv_heads=2, head_dim=8,
                     density=0.5, dtype="fp16")
    o, lse = ora.bsr_attention(w.q, w.k, w.v, w.R, w.C, w.indptr, w.indices, "fp16", 2)
    Q = ora.storage_to_f64(w.q, "fp16")
    K = ora.storage_to_f64(w.k, "fp16")
    V = ora.storage_to_f64(w.v, "fp16")
    scale = 1 / math.sqrt(8)
    for i in range(w.M):
        rb = i // w.R
        cols = set(int(c) for c in w.indices[w.indptr[rb]:w.indptr[rb + 1]])
        for hq in range(4):
            h = hq // 2
            keys = [t for t in range(w.N) if t // w.C in cols]
            if not keys:
                assert lse[i, hq] == -math.inf and np.all(o[i, hq] == 0)
                continue
            s = [scale * sum(Q[i, hq, j] * K[t, h, j] for j in range(8)) for t in keys]
            z = sum(math.exp(x) for x in s)
            ref_o = sum(math.exp(x) / z * V[t, h] for x, t in zip(s, keys))
            assert abs(lse[i, hq] - math.log(z)) < 1e-12
            assert np.max(np.abs(o[i, hq] - ref_o)) < 1e-12


def test_bsr_vector_sparse_matches_sdpa_with_mask():
    # R = C = 1: an arbitrary element mask; torch SDPA with a boolean mask
    rng = np.random.Generator(np.random.PCG64(5))
    M, N, d = 9, 11, 16
    dense = rng.random((M, N)) < 0.35
    dense[:, 0] |= ~dense.any(axis=1)           # every row sees at least one key
    indptr = np.concatenate([[0], np.cumsum(dense.sum(axis=1))]).astype(np.int32)
    indices = np.concatenate([np.nonzero(r)[0] for r in dense]).astype(np.int32)
    q = wl.normal_bits(rng, (M, 2, d), "bf16")
    k = wl.normal_bits(rng, (N, 1, d), "bf16")
    v = wl.normal_bits(rng, (N, 1, d), "bf16")
    o, _ = ora.bsr_attention(q, k, v, 1, 1, indptr, indices, "bf16", 1)
    for hq in range(2):
        ref = _sdpa(ora.storage_to_f64(q[:, hq], "bf16"), ora.storage_to_f64(k[:, 0], "bf16"),
                    ora.storage_to_f64(v[:, 0], "bf16"), 1 / math.sqrt(d), dense)
        assert np.max(np.abs(o[:, hq] - ref)) < 1e-12


def test_bsr_full_and_block_diagonal_masks():
    rng = np.random.Generator(np.random.PCG64(6))
    M, N, R, C, d = 8, 8, 4, 4, 16
    q = wl.normal_bits(rng, (M, 4, d), "bf16")
    k = wl.normal_bits(rng, (N, 2, d), "bf16")
    v = wl.normal_bits(rng, (N, 2, d), "bf16")
    Q = ora.storage_to_f64(q, "bf16")
    K = ora.storage_to_f64(k, "bf16")
    V = ora.storage_to_f64(v, "bf16")
    sc = 1 / math.sqrt(d)
    # every block listed: plain dense attention (GQA: qo head h reads kv head h // 2)
    o, _ = ora.bsr_attention(q, k, v, R, C, [0, 2, 4], [0, 1, 0, 1], "bf16", 2)
    for hq in range(4):
        assert np.max(np.abs(o[:, hq] - _sdpa(Q[:, hq], K[:, hq // 2], V[:, hq // 2], sc))) < 1e-12
    # block diagonal: each half attends only to its own half
    o, _ = ora.bsr_attention(q, k, v, R, C, [0, 1, 2], [0, 1], "bf16", 2)
    for hq in range(4):
        h = hq // 2
        for b in range(2):
            sl = slice(4 * b, 4 * b + 4)
            ref = _sdpa(Q[sl, hq], K[sl, h], V[sl, h], sc)
            assert np.max(np.abs(o[sl, hq] - ref)) < 1e-12


def test_bsr_equals_paged_append_over_the_blocks():
    # a row block of the BSR mask is an append "request" whose pages are the
    # listed column blocks: the paged (non-causal) oracle must agree
    w = wl.small_bsr(12, M=10, N=16, R=4, C=4, num_qo_heads=4, num_kv_heads=2, head_dim=8,
                     density=0.5)
    o, lse = ora.bsr_attention(w.q, w.k, w.v, w.R, w.C, w.indptr, w.indices, "bf16", 2)
    nrb = len(w.indptr) - 1
    qo_indptr = np.minimum(np.arange(nrb + 1) * w.R, w.M)
    pages_k = w.k.reshape(w.N // w.C, w.C, 2, 8)
    pages_v = w.v.reshape(w.N // w.C, w.C, 2, 8)
    lpl = np.full(nrb, w.C)
    o2, lse2 = ora.paged_append(w.q, qo_indptr, pages_k, pages_v, w.indptr, w.indices, lpl,
                                w.C, "bf16", 2, causal=False)
    assert np.max(np.abs(o - o2)) < 1e-12
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse2))
    fin = np.isfinite(lse)
    assert np.max(np.abs(lse[fin] - lse2[fin])) < 1e-12


def test_bsr_empty_row_block():
    w = wl.small_bsr(13, M=8, N=8, R=4, C=2, num_qo_heads=2, num_kv_heads=2, head_dim=8,
                     empty_rows={1})
    o, lse = ora.bsr_attention(w.q, w.k, w.v, w.R, w.C, w.indptr, w.indices, "bf16", 2)
    assert np.all(np.isneginf(lse[4:])) and np.all(o[4:] == 0)
    assert np.all(np.isfinite(lse[:4]))


# ----------------------------------------------------------------------------
# page append
# ----------------------------------------------------------------------------
def test_append_paged_kv_hand_example():
    # page size 2, pool of 4 pages (value = 100 + 10 * page + slot).
    # request 0: pages [3, 1], 3 tokens, the last 2 are new -> positions 1, 2:
    #   new row 0 -> page 3 slot 1, new row 1 -> page 1 slot 0.
    # request 1: page [0], 2 tokens, 1 new -> position 1: new row 2 -> page 0 slot 1.
    # page 2 and the other slots keep their values.
    P = 2
    pool = (100 + 10 * np.arange(4)[:, None] + np.arange(P)[None, :]).astype(np.int64)[:, :, None, None]
    new = np.array([7, 8, 9], dtype=np.int64)[:, None, None]
    kp, vp = ora.append_paged_kv(new, -new, [0, 2, 3], pool, pool, [0, 2, 3], [3, 1, 0], [1, 2], P)
    want = pool.copy()
    want[3, 1] = 7
    want[1, 0] = 8
    want[0, 1] = 9
    assert np.array_equal(kp, want)
    wantv = pool.copy()
    wantv[3, 1] = -7
    wantv[1, 0] = -8
    wantv[0, 1] = -9
    assert np.array_equal(vp, wantv)


@pytest.mark.parametrize("P", [1, 3, 16])
def test_append_then_walk_returns_new_rows(P):
    kv_lens = [0, 5, 40, 17, 1]
    app = [0, 5, 7, 1, 1]
    w = wl.page_append(30 + P, kv_lens, app, P, 2, head_dim=8)
    kv = w.kv
    kp, vp = ora.append_paged_kv(w.k_new, w.v_new, w.append_indptr, kv.k_pages, kv.v_pages,
                                 kv.kv_indptr, kv.kv_indices, kv.kv_last_page_len, P)
    changed = 0
    for b, (L, n) in enumerate(zip(kv_lens, app)):
        a0 = int(w.append_indptr[b])
        rows_k = ora.walk_pages(kp, kv.kv_indptr, kv.kv_indices, kv.kv_last_page_len, P, b)
        rows_v = ora.walk_pages(vp, kv.kv_indptr, kv.kv_indices, kv.kv_last_page_len, P, b)
        old_k = ora.walk_pages(kv.k_pages, kv.kv_indptr, kv.kv_indices, kv.kv_last_page_len, P, b)
        assert np.array_equal(rows_k[L - n:], w.k_new[a0:a0 + n])
        assert np.array_equal(rows_v[L - n:], w.v_new[a0:a0 + n])
        assert np.array_equal(rows_k[:L - n], old_k[:L - n])
        changed += n
    # nothing outside the appended slots moved (extra pages included)
    diff = np.any(kp != kv.k_pages, axis=(2, 3)).sum()
    assert diff <= changed


def test_append_skips_positions_outside_the_request():
    # 3 new rows for a request of 2 tokens: the first would sit at position -1
    w = wl.page_append(40, [2], [2], 4, 1, head_dim=8)
    kv = w.kv
    k_new = np.concatenate([w.k_new[:1], w.k_new])
    ai = np.array([0, 3], dtype=np.int32)
    kp, _ = ora.append_paged_kv(k_new, k_new, ai, kv.k_pages, kv.v_pages, kv.kv_indptr,
                                kv.kv_indices, kv.kv_last_page_len, 4)
    rows = ora.walk_pages(kp, kv.kv_indptr, kv.kv_indices, kv.kv_last_page_len, 4, 0)
    assert np.array_equal(rows, k_new[1:])


# ----------------------------------------------------------------------------
# LLaMA 3.1 RoPE frequency scaling
# ----------------------------------------------------------------------------
L31 = (8.0, 1.0, 4.0, 8192.0)   # the published LLaMA 3.1 settings


def test_llama31_identity_and_bounds():
    f = ora.rope_inv_freq(128, 500000.0)
    # factor 1: every band gives the plain frequency (the blend up to rounding)
    assert np.allclose(ora.rope_inv_freq(128, 500000.0, (1.0, 1.0, 4.0, 8192.0)), f,
                       rtol=1e-15, atol=0)
    g = ora.rope_inv_freq(128, 500000.0, L31)
    r = g / f
    assert np.all(r <= 1.0) and np.all(r >= 1 / 8.0 - 1e-15)
    assert np.all(np.diff(r) <= 0)               # stronger scaling at longer wavelengths
    assert r[0] == 1.0 and r[-1] == 1 / 8.0        # wavelength 2 pi: kept; ~2.4e6: divided
    # with theta 500000, d 128: 29 pairs kept, 6 blended, 29 divided
    assert (r == 1.0).sum() == 29 and (r == 1 / 8.0).sum() == 29


@pytest.mark.parametrize("edge", ["high", "low"])
def test_llama31_continuous_at_band_edges(edge):
    # choose theta so that pair 1's wavelength sits just inside the blended band
    # at one edge: the blended value must approach the neighbouring band's value
    factor, low, high, old = L31
    w_edge = old / high if edge == "high" else old / low
    for eps in (1e-3, 1e-6):
        w = w_edge * (1 + eps) if edge == "high" else w_edge * (1 - eps)
        # wavelength of pair j=1 at head_dim 4 is 2 pi * theta^(1/2)
        theta = (w / (2 * math.pi)) ** 2
        f = ora.rope_inv_freq(4, theta)[1]
        g = ora.rope_inv_freq(4, theta, L31)[1]
        limit = f if edge == "high" else f / factor
        assert abs(g - limit) / limit < 10 * eps


def test_llama31_rotation_keeps_norms_and_relative_positions():
    x = np.random.Generator(np.random.PCG64(7)).standard_normal((5, 128))
    y = np.random.Generator(np.random.PCG64(8)).standard_normal((5, 128))
    pos = np.array([0, 1, 100, 4097, 65535])
    xr = ora.rope_rotate(x, pos, 500000.0, L31)
    assert np.allclose(np.linalg.norm(xr, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    # logits depend only on the position difference
    a = (ora.rope_rotate(x, 10, 5e5, L31) * ora.rope_rotate(y, 3, 5e5, L31)).sum(-1)
    b = (ora.rope_rotate(x, 5010, 5e5, L31) * ora.rope_rotate(y, 5003, 5e5, L31)).sum(-1)
    assert np.allclose(a, b, rtol=1e-9, atol=1e-9)
    assert np.array_equal(ora.rope_rotate(x, 0, 5e5, L31), x)


# ----------------------------------------------------------------------------
# fp8 (OCP e4m3) KV cache
# ----------------------------------------------------------------------------
def test_fp8_e4m3_constants():
    # values fixed by the OCP FP8 E4M3 definition (bias 7, no infinity)
    codes = [0x00, 0x01, 0x07, 0x08, 0x38, 0x3C, 0xB8, 0xC0, 0x7E, 0xFE, 0x77]
    want = [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.5, -1.0, -2.0, 448.0, -448.0,
            240.0]
    got = ora.fp8_e4m3_to_f64(np.array(codes, np.uint8))
    assert list(got) == want
    assert np.isnan(ora.fp8_e4m3_to_f64(np.array([0x7F, 0xFF], np.uint8))).all()


def test_fp8_e4m3_all_codes_match_torch():
    # library special case: torch's float8_e4m3fn over all 256 codes
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = ora.fp8_e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])


def test_fp8_decode_equals_decode_on_the_same_values():
    # fp8 pages with scales equal a 16-bit cache holding scale * value exactly
    # (e4m3 values times a power of two are exact in bf16)
    w = wl.small_decode_fp8(50, [1, 33, 300], 16, 8, 2, k_scale=0.25, v_scale=2.0)
    o, lse = ora.decode_workload(w)
    kv = w.kv
    kb = wl.round_to_bf16_bits(
        (0.25 * ora.fp8_e4m3_to_f64(kv.k_pages)).astype(np.float32))
    vb = wl.round_to_bf16_bits((2.0 * ora.fp8_e4m3_to_f64(kv.v_pages)).astype(np.float32))
    assert np.array_equal(ora.storage_to_f64(kb, "bf16"), 0.25 * ora.fp8_e4m3_to_f64(kv.k_pages))
    o2, lse2 = ora.paged_decode(w.q, kb, vb, kv.kv_indptr, kv.kv_indices, kv.kv_last_page_len,
                                16, "bf16", 2)
    assert np.max(np.abs(o - o2)) < 1e-12 and np.max(np.abs(lse - lse2)) < 1e-12
    # the scales act as stated: k_scale multiplies every logit, v_scale every output
    w1 = wl.small_decode_fp8(50, [1, 33, 300], 16, 8, 2, k_scale=1.0, v_scale=1.0)
    o1, _ = ora.decode_workload(w1)
    w3 = wl.small_decode_fp8(50, [1, 33, 300], 16, 8, 2, k_scale=1.0, v_scale=3.0)
    o3, _ = ora.decode_workload(w3)
    assert np.max(np.abs(3.0 * o1 - o3)) < 1e-12


# ----------------------------------------------------------------------------
# interleaved (adjacent-pair) RoPE
# ----------------------------------------------------------------------------
def test_interleaved_rope_is_complex_multiplication():
    # adjacent pairs as complex numbers, multiplied by exp(i * pos * f_j)
    x = np.random.Generator(np.random.PCG64(60)).standard_normal((3, 128))
    pos = np.array([0.0, 7.0, 5000.0])
    f = ora.rope_inv_freq(128, 5e5)
    z = (x[:, 0::2] + 1j * x[:, 1::2]) * np.exp(1j * pos[:, None] * f)
    want = np.empty_like(x)
    want[:, 0::2], want[:, 1::2] = z.real, z.imag
    got = ora.rope_rotate(x, pos, 5e5, interleave=True)
    assert np.max(np.abs(got - want)) < 1e-12


def test_interleaved_rope_is_rotate_half_on_deinterleaved_elements():
    # de-interleaving (evens first, then odds) maps adjacent pairs to (j, j + d/2)
    x = np.random.Generator(np.random.PCG64(61)).standard_normal((4, 128))
    perm = np.concatenate([np.arange(0, 128, 2), np.arange(1, 128, 2)])
    for l31 in (None, (8.0, 1.0, 4.0, 8192.0)):
        a = ora.rope_rotate(x, 321.0, 5e5, l31, interleave=True)
        b = ora.rope_rotate(x[:, perm], 321.0, 5e5, l31)
        assert np.max(np.abs(a[:, perm] - b)) < 1e-12


def test_interleaved_rope_attention_equals_rotate_half_on_permuted_heads():
    # attention with interleaved RoPE == rotate-half RoPE after the same
    # element permutation of q and k (logits are permutation invariant)
    w = wl.small_decode(62, [5, 90], 16, 4, 2, head_dim=128)
    w.rope_theta = 5e5
    w.rope_interleave = True
    o1, l1 = ora.decode_workload(w)
    perm = np.concatenate([np.arange(0, 128, 2), np.arange(1, 128, 2)])
    w2 = wl.small_decode(62, [5, 90], 16, 4, 2, head_dim=128)
    w2.rope_theta = 5e5
    w2.q = w2.q[..., perm]
    w2.kv.k_pages = w2.kv.k_pages[..., perm]
    o2, l2 = ora.decode_workload(w2)
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12
