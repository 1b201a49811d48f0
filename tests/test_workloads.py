"""CPU checks of the input generators that the parity tests rely on."""
import numpy as np
import pytest

from attention_bsr_paged_amd import workloads as wl
from oracle import attention as ora


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp8_e4m3"])
@pytest.mark.parametrize("P", [1, 3, 16])
def test_poison_unwritten_changes_only_slots_without_a_token(dtype, P):
    rng = np.random.Generator(np.random.PCG64(17 + P))
    lens = [0, 1, P, P + 1, 5 * P - 1, 40]
    kv = wl.make_paged_kv(rng, lens, P, 2, 8, "bf16", extra_pages=3)
    if dtype == "fp16":
        kv = wl.make_paged_kv(rng, lens, P, 2, 8, "fp16", extra_pages=3)
    elif dtype == "fp8_e4m3":
        kv = wl.to_fp8_kv(rng, kv, 1.0)
    bad = wl.poison_unwritten(kv)
    valid = np.zeros(kv.k_pages.shape[:2], dtype=bool)      # [page, slot]
    for b in range(len(lens)):
        for t in range(lens[b]):
            valid[kv.kv_indices[kv.kv_indptr[b] + t // P], t % P] = True
    for pool, pois in ((kv.k_pages, bad.k_pages), (kv.v_pages, bad.v_pages)):
        assert np.array_equal(pool[valid], pois[valid])
        vals = ora.storage_to_f64(pois[~valid], dtype)
        assert not np.isfinite(vals).any()
        assert np.isnan(vals).any()
    # the oracle reads valid slots only: same results on either cache
    q = wl.normal_bits(rng, (len(lens), 4, 8), "bf16" if dtype != "fp16" else "fp16")
    qd = "fp16" if dtype == "fp16" else "bf16"
    a = ora.paged_decode(q, kv.k_pages, kv.v_pages, kv.kv_indptr, kv.kv_indices,
                         kv.kv_last_page_len, P, qd, 2, kv_dtype=kv.dtype)
    c = ora.paged_decode(q, bad.k_pages, bad.v_pages, bad.kv_indptr, bad.kv_indices,
                         bad.kv_last_page_len, P, qd, 2, kv_dtype=kv.dtype)
    assert np.array_equal(a[0], c[0]) and np.array_equal(a[1], c[1])
