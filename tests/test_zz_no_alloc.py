"""The no-allocation batch decode (abp_decode_static) through the C ABI: its
output must equal the plan + run entry points' bit for bit at the same worker
count, and meet the parity bar against the oracle, on two calls in a row (the
second with a smaller batch, so it runs on what the first left in the
library's scratch)."""
import ctypes

import numpy as np
import pytest

import attention_bsr_paged_amd as abp
from attention_bsr_paged_amd import workloads as wl
from oracle import attention as ora

from gpu_helpers import assert_parity, run_decode, say, torch_dtype, upload_kv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    abp.load_library()


def decode_static(w, num_workers):
    import torch
    lib = abp.load_library()
    kv = w.kv
    dev = upload_kv(kv)
    q = wl.to_torch(w.q, w.dtype, "cuda")
    dt = torch_dtype(w.dtype)
    params = abp.make_params(w.num_qo_heads, w.num_kv_heads, w.head_dim, kv.page_size, dt)
    o = torch.full(q.shape, float("nan"), dtype=dt, device="cuda")
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    indptr = np.ascontiguousarray(kv.kv_indptr, np.int32)
    lpl = np.ascontiguousarray(kv.kv_last_page_len, np.int32)
    stream = torch.cuda.current_stream()
    st = lib.abp_decode_static(ctypes.byref(params), w.batch, indptr.ctypes.data, lpl.ctypes.data,
                               num_workers, q.data_ptr(), dev["k"].data_ptr(),
                               dev["v"].data_ptr(), dev["indptr"].data_ptr(),
                               dev["indices"].data_ptr(), dev["lpl"].data_ptr(), None, None,
                               o.data_ptr(), lse.data_ptr(), ctypes.c_void_p(stream.cuda_stream))
    assert st == abp.ABP_OK, abp.abp_last_error()
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


def test_decode_static_equals_plan_run_on_two_calls():
    big = wl.batch_decode_gqa()                                  # 64 requests, GQA 32/8
    small = wl.small_decode(61, [0, 1, 17, 300, 2049], 16, 32, 8)  # then a smaller batch
    for w, W in ((big, 256), (small, 7)):
        say(f"[case] abp_decode_static {w.name} W={W}")
        o, l = decode_static(w, W)
        o2, l2 = run_decode(w, num_workers=W)
        assert np.array_equal(o, o2) and np.array_equal(l, l2), f"{w.name}: differs from plan + run"
        o_ref, l_ref = ora.decode_workload(w)
        assert_parity(o, l, o_ref, l_ref, w.dtype, what=f"abp_decode_static {w.name}")


def test_decode_static_default_workers_and_repeat():
    w = wl.small_decode(62, [5, 77, 1500, 4096], 16, 32, 8)
    o_ref, l_ref = ora.decode_workload(w)
    first = decode_static(w, 0)
    assert_parity(*first, o_ref, l_ref, w.dtype, what="abp_decode_static default workers")
    again = decode_static(w, 0)
    assert np.array_equal(first[0], again[0]) and np.array_equal(first[1], again[1])
