"""Pins of the oracle's RoPE append branch (CPU only).

The append oracle rotates query i of a request (qo_len queries, kv_len keys)
at position kv_len - qo_len + i unless positions are given, and key t at
kv_pos_offset + t. Two pins fix those positions from outside the branch:

- a closed form: with every key zero except one, each row's lse and o follow
  from a single logit, which is computed here from the complex-number form of
  the rotation (pair j of x is the complex number z_j, rotation by angle a
  multiplies it by exp(i a), and <x, y> = Re sum_j z_j(x) conj(z_j(y))). Only
  the position difference enters, so an off-by-one in either position moves
  every logit of the high-frequency pairs;
- the causal identity: row i of a causal RoPE append equals a RoPE decode over
  the first kv_len - qo_len + i + 1 keys, whose query sits on its last key.

Both run for the rotate-half pairing, the interleaved pairing and the LLaMA 3.1
frequencies.
"""
import math

import numpy as np
import pytest

from oracle import attention as ora
from attention_bsr_paged_amd import workloads as wl

THETA = 500000.0
L31 = (8.0, 1.0, 4.0, 8192.0)
VARIANTS = [("rotate_half", None, False), ("interleaved", None, True), ("llama31", L31, False)]


def _complex_pairs(x, interleave):
    x = np.asarray(x, np.float64)
    h = x.shape[-1] // 2
    if interleave:
        return x[..., 0::2] + 1j * x[..., 1::2]
    return x[..., :h] + 1j * x[..., h:]


def _set_logical(pages, kv, b, t, value_bits):
    """Write one logical token row (all kv heads) of request b into a pool."""
    P = kv.page_size
    page = int(kv.kv_indices[int(kv.kv_indptr[b]) + t // P])
    pages[page, t % P] = value_bits


@pytest.mark.parametrize("name,l31,il", VARIANTS)
@pytest.mark.parametrize("off", [0, 37])
def test_rope_append_single_key_closed_form(name, l31, il, off):
    d, Hkv, G, P = 16, 1, 2, 4
    E, n = 9, 7                         # existing keys, new query tokens
    i0 = 2                              # the nonzero key is row i0's last visible key
    w = wl.small_append(300 + off, [n], [E + n], P, Hkv * G, Hkv, head_dim=d, causal=True)
    kv = w.kv
    rng = np.random.Generator(np.random.PCG64(301 + off))
    kv.k_pages[:] = 0
    kv.v_pages[:] = 0
    j_star = E + i0
    k_bits = wl.normal_bits(rng, (Hkv, d), "bf16")
    u_bits = wl.normal_bits(rng, (Hkv, d), "bf16")
    _set_logical(kv.k_pages, kv, 0, j_star, k_bits)
    _set_logical(kv.v_pages, kv, 0, j_star, u_bits)
    kv_off = np.array([off], np.int32)
    o, lse = ora.paged_append(w.q, w.qo_indptr, kv.k_pages, kv.v_pages, kv.kv_indptr,
                              kv.kv_indices, kv.kv_last_page_len, P, "bf16", Hkv, causal=True,
                              rope_theta=THETA, kv_pos_offset=kv_off, rope_llama31=l31,
                              rope_interleave=il)
    f = ora.rope_inv_freq(d, THETA, l31)
    scale = 1.0 / math.sqrt(d)
    k = ora.storage_to_f64(k_bits, "bf16")[0]
    u = ora.storage_to_f64(u_bits, "bf16")[0]
    zk = _complex_pairs(k, il)
    for i in range(n):
        nvis = E + i + 1                     # keys 0 .. E + i
        for g in range(G):
            q = ora.storage_to_f64(w.q[i, g], "bf16")
            if i < i0:
                # every visible key is zero: n equal logits of 0, and no value
                assert lse[i, g] == pytest.approx(math.log(nvis), abs=1e-12)
                assert np.all(o[i, g] == 0)
                continue
            # query at E + i, the key at off + E + i0: the difference is i - i0 - off
            delta = (i - i0) - off
            s = scale * np.real(np.sum(_complex_pairs(q, il) * np.conj(zk) * np.exp(1j * delta * f)))
            want_lse = math.log((nvis - 1) + math.exp(s))
            assert lse[i, g] == pytest.approx(want_lse, abs=1e-12), (name, i, g)
            assert np.allclose(o[i, g], math.exp(s - want_lse) * u, atol=1e-12), (name, i, g)


def test_rope_single_key_detects_a_shifted_query_position():
    """The closed form above separates neighbouring positions: the logit of the
    one nonzero key moves by far more than the tolerance between delta and delta + 1."""
    d = 16
    f = ora.rope_inv_freq(d, THETA)
    rng = np.random.Generator(np.random.PCG64(7))
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    s = [np.real(np.sum(_complex_pairs(q, False) * np.conj(_complex_pairs(k, False))
                        * np.exp(1j * dl * f))) for dl in (0, 1)]
    assert abs(s[0] - s[1]) > 1e-2


@pytest.mark.parametrize("name,l31,il", VARIANTS)
@pytest.mark.parametrize("off", [0, 500])
def test_rope_causal_row_equals_rope_decode_over_its_prefix(name, l31, il, off):
    d, Hkv, G, P = 16, 2, 2, 4
    w = wl.small_append(310 + off, [6, 3], [19, 3], P, Hkv * G, Hkv, head_dim=d, causal=True)
    kv = w.kv
    kv_off = np.array([off, off + 11], np.int32)
    o, l = ora.paged_append(w.q, w.qo_indptr, kv.k_pages, kv.v_pages, kv.kv_indptr,
                            kv.kv_indices, kv.kv_last_page_len, P, "bf16", Hkv, causal=True,
                            rope_theta=THETA, kv_pos_offset=kv_off, rope_llama31=l31,
                            rope_interleave=il)
    for b in range(2):
        q0, q1 = int(w.qo_indptr[b]), int(w.qo_indptr[b + 1])
        qo_len, kv_len = q1 - q0, int(kv.kv_len[b])
        pages = kv.kv_indices[kv.kv_indptr[b]:kv.kv_indptr[b + 1]]
        for i in range(qo_len):
            nk = kv_len - qo_len + i + 1
            npg = -(-nk // P)
            # decode over the truncated table; its default query position is nk - 1
            od, ld = ora.paged_decode(w.q[q0 + i:q0 + i + 1], kv.k_pages, kv.v_pages,
                                      np.array([0, npg]), pages[:npg],
                                      np.array([nk - (npg - 1) * P]), P, "bf16", Hkv,
                                      rope_theta=THETA, kv_pos_offset=kv_off[b:b + 1],
                                      rope_llama31=l31, rope_interleave=il)
            assert np.allclose(o[q0 + i], od[0], atol=1e-13), (name, b, i)
            assert np.allclose(l[q0 + i], ld[0], atol=1e-13), (name, b, i)


def test_rope_decode_single_key_closed_form():
    """Decode: the query sits on the last key (kv_len - 1), so a request whose
    only nonzero key is its last one has the unrotated logit when the key offset
    is 0, for any position of that key."""
    d, Hkv, G, P = 16, 1, 1, 4
    for kv_len in (1, 5, 13):
        w = wl.small_decode(320 + kv_len, [kv_len], P, Hkv * G, Hkv, head_dim=d)
        kv = w.kv
        kv.k_pages[:] = 0
        kv.v_pages[:] = 0
        rng = np.random.Generator(np.random.PCG64(kv_len))
        k_bits = wl.normal_bits(rng, (Hkv, d), "bf16")
        u_bits = wl.normal_bits(rng, (Hkv, d), "bf16")
        _set_logical(kv.k_pages, kv, 0, kv_len - 1, k_bits)
        _set_logical(kv.v_pages, kv, 0, kv_len - 1, u_bits)
        o, lse = ora.paged_decode(w.q, kv.k_pages, kv.v_pages, kv.kv_indptr, kv.kv_indices,
                                  kv.kv_last_page_len, P, "bf16", Hkv, rope_theta=THETA)
        q = ora.storage_to_f64(w.q[0, 0], "bf16")
        s = float(q @ ora.storage_to_f64(k_bits[0], "bf16")) / math.sqrt(d)
        want = math.log((kv_len - 1) + math.exp(s))
        assert lse[0, 0] == pytest.approx(want, abs=1e-12)
        assert np.allclose(o[0, 0], math.exp(s - want) * ora.storage_to_f64(u_bits[0], "bf16"),
                           atol=1e-12)
