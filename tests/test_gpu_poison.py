"""GPU parity with non-finite bits in every slot that holds no token.

The page table defines only the first kv_last_page_len slots of a request's
last page; the other slots of that page, and every page no request owns, may
hold any bits (a cache allocated without clearing, or reused). Here they hold
NaN / inf patterns of the storage type (e4m3: its NaN codes), and every path
must still meet the parity bar against the oracle, which reads valid slots
only. The kernels' fast paths load whole 4- or 16-row groups; rows past a
request's end must never reach the P.V products, where p = 0 would not cancel
a NaN.

Block-sparse attention is not listed: its K/V are dense ([N, Hkv, d] with N a
multiple of the column block), so it has no slot without a key.
"""
import numpy as np
import pytest

import attention_bsr_paged_amd as abp
from attention_bsr_paged_amd import workloads as wl
from oracle import attention as ora

from gpu_helpers import assert_parity, run_append, run_decode, say

pytestmark = pytest.mark.gpu

# lengths chosen so that most last pages are partial at page sizes 3, 16 and 256
DEC_LENS = [0, 1, 15, 17, 63, 65, 200, 1000, 2501]
QO = [1, 5, 31, 33, 64, 130, 300]
KV_EXTRA = [0, 3, 1, 200, 17, 1000, 65]


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    abp.load_library()


def _poison(w):
    w.kv = wl.poison_unwritten(w.kv)
    return w


@pytest.mark.parametrize("P,G,hkv", [(16, 4, 8), (16, 8, 4), (256, 4, 4),   # matrix-core decode
                                     (16, 2, 2), (3, 4, 2), (16, 1, 8)])     # vector-unit decode
def test_decode_poisoned_unwritten_slots(P, G, hkv):
    say(f"[case] poisoned decode P={P} G={G} hkv={hkv}")
    w = _poison(wl.small_decode(900 + P + G + hkv, DEC_LENS, P, G * hkv, hkv, extra_pages=4))
    o_ref, l_ref = ora.decode_workload(w)
    for W in (1, 13, 0):
        o, l = run_decode(w, num_workers=W)
        assert_parity(o, l, o_ref, l_ref, "bf16", what=f"poisoned decode P{P} G{G} W{W}")


@pytest.mark.parametrize("P,G,hkv,dtype", [(16, 4, 8, "bf16"), (16, 8, 4, "fp16"),   # matrix cores
                                           (16, 2, 2, "bf16"), (3, 4, 2, "fp16")])   # vector unit
def test_fp8_decode_poisoned_unwritten_slots(P, G, hkv, dtype):
    say(f"[case] poisoned fp8 decode P={P} G={G} hkv={hkv} q {dtype}")
    w = _poison(wl.small_decode_fp8(910 + P + G + hkv, DEC_LENS, P, G * hkv, hkv, dtype=dtype))
    o_ref, l_ref = ora.decode_workload(w)
    for W in (1, 0):
        o, l = run_decode(w, num_workers=W)
        assert_parity(o, l, o_ref, l_ref, dtype, what=f"poisoned fp8 decode P{P} G{G} W{W}")


@pytest.mark.parametrize("rope", [False, True])
@pytest.mark.parametrize("P", [3, 16])
def test_rope_decode_poisoned(rope, P):
    say(f"[case] poisoned decode rope={rope} P={P}")
    w = _poison(wl.small_decode(920 + P, DEC_LENS, P, 8, 2, extra_pages=2))
    if rope:
        w.rope_theta = 500000.0
        w.kv_pos_offset = np.arange(len(DEC_LENS), dtype=np.int32) * 7
        w.q_pos = (w.kv_pos_offset + w.kv.kv_len - 1).astype(np.int32)
    o_ref, l_ref = ora.decode_workload(w)
    o, l = run_decode(w, num_workers=11)
    assert_parity(o, l, o_ref, l_ref, "bf16", what=f"poisoned decode rope={rope} P{P}")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("rope", [False, True])
@pytest.mark.parametrize("P", [3, 16, 256])
def test_append_poisoned_unwritten_slots(causal, rope, P):
    say(f"[case] poisoned append causal={causal} rope={rope} P={P}")
    kv = [q + e for q, e in zip(QO, KV_EXTRA)]
    w = _poison(wl.small_append(930 + P + 2 * rope + causal, QO, kv, P, 8, 2, causal=causal,
                                extra_pages=3))
    if rope:
        w.rope_theta = 500000.0
    o_ref, l_ref = ora.append_workload(w)
    for W in (1, 9, 0):
        o, l = run_append(w, num_workers=W)
        assert_parity(o, l, o_ref, l_ref, "bf16",
                      what=f"poisoned append c{int(causal)} rope{int(rope)} P{P} W{W}")


def test_cascade_poisoned():
    """Both levels poisoned: a prefix of 700 tokens (last page of 256 partial) and
    suffixes in pages of 16, with and without RoPE."""
    from test_gpu_append import run_cascade, small_cascade
    for theta in (0.0, 500000.0):
        say(f"[case] poisoned cascade theta={theta}")
        w = small_cascade(940, theta)
        w.prefix = wl.poison_unwritten(w.prefix)
        w.kv = wl.poison_unwritten(w.kv)
        o_ref, l_ref = ora.decode_workload(w)
        o, l = run_cascade(w, num_workers=9, prefix_workers=4)
        assert_parity(o, l, o_ref, l_ref, "bf16", what=f"poisoned cascade theta={theta}")


@pytest.mark.parametrize("causal", [True, False])
def test_pod_poisoned(causal):
    from test_gpu_pod import run_pod
    say(f"[case] poisoned mixed batch causal={causal}")
    dec = _poison(wl.small_decode(950, [0, 1, 15, 17, 300, 1000, 2049], 16, 16, 4))
    app = _poison(wl.small_append(951, [1, 37, 128, 200], [5, 100, 301, 700], 16, 16, 4,
                                  causal=causal))
    w = wl.mixed_batch(dec, app, "poisoned_mixed")
    for groups, dgroups in ((0, 0), (5, 2)):
        (od, ld), (oa, la), _ = run_pod(w, groups, dgroups)
        od_ref, ld_ref = ora.decode_workload(w.dec)
        oa_ref, la_ref = ora.append_workload(w.app)
        assert_parity(od, ld, od_ref, ld_ref, "bf16", what=f"poisoned pod decode g{groups}")
        assert_parity(oa, la, oa_ref, la_ref, "bf16", what=f"poisoned pod append g{groups}")
