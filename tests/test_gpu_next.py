"""GPU checks of the block-sparse attention path, the page-append kernel and
LLaMA 3.1 RoPE against the fp64 oracle, through the C ABI.

- Block-sparse attention is compared element by element on small patterns
  (several tiles, ragged last row block, empty row blocks, block sizes 1 to 64)
  and on sampled rows of the benchmark's 8192 x 8192 pattern in its launch
  configuration.
- Page append is compared bit for bit over whole page pools.
- LLaMA 3.1 RoPE decode, append and cascade are compared to the parity bar.
"""
import numpy as np
import pytest

import attention_bsr_paged_amd as abp
from attention_bsr_paged_amd import workloads as wl
from oracle import attention as ora

from gpu_helpers import (assert_parity, i32, run_append, run_bsr, run_decode, say, torch_dtype,
                         upload_kv)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    abp.load_library()


# ----------------------------------------------------------------------------
# block-sparse attention
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("R,C", [(1, 1), (16, 3), (64, 16), (100, 64), (7, 16), (64, 1)])
@pytest.mark.parametrize("G", [1, 4])
def test_small_bsr_parity(R, C, G):
    ncb = max(1, 384 // C)
    M = 333
    say(f"[case] bsr R={R} C={C} G={G}")
    w = wl.small_bsr(400 + R + C + G, M, ncb * C, R, C, 2 * G, 2, density=0.3,
                     empty_rows={1})
    o_ref, l_ref = ora.bsr_attention(w.q, w.k, w.v, R, C, w.indptr, w.indices, "bf16", 2)
    for W in (1, 13, 0):
        o, l = run_bsr(w, num_workers=W)
        assert_parity(o, l, o_ref, l_ref, "bf16", what=f"bsr R{R} C{C} G{G} W{W}")


def test_bsr_fp16_dense_pattern_and_f32_out():
    w = wl.small_bsr(410, 200, 256, 32, 16, 16, 2, density=1.0, dtype="fp16")
    o_ref, l_ref = ora.bsr_attention(w.q, w.k, w.v, w.R, w.C, w.indptr, w.indices, "fp16", 2)
    o, l = run_bsr(w, num_workers=7)
    assert_parity(o, l, o_ref, l_ref, "fp16", what="bsr fp16 dense")
    import torch
    o32, l32 = run_bsr(w, num_workers=7, out_dtype=torch.float32)
    assert_parity(o32, l32, o_ref, l_ref, "fp16", what="bsr fp16 -> f32")


def test_bsr_replan_and_determinism():
    """One runner, two patterns in turn; each result bit-identical on a rerun."""
    import torch
    w1 = wl.small_bsr(420, 256, 512, 64, 16, 32, 8, density=0.4)
    w2 = wl.small_bsr(421, 130, 512, 16, 16, 32, 8, density=0.1, empty_rows={0, 3})
    params = abp.make_params(32, 8, 128, 16, torch.bfloat16)
    runner = abp.BlockSparseAttention(params, max_row_blocks=16, max_M=256, num_workers=29)
    for w in (w1, w2, w1):
        o_ref, l_ref = ora.bsr_attention(w.q, w.k, w.v, w.R, w.C, w.indptr, w.indices, "bf16", 8)
        o, l = run_bsr(w, runner=runner)
        o2, l2 = run_bsr(w, runner=runner)
        assert_parity(o, l, o_ref, l_ref, "bf16", what=f"bsr replan {w.name}")
        assert np.array_equal(o, o2) and np.array_equal(l, l2)


def test_bsr_full_sampled():
    """The benchmark's pattern (8192 x 8192, R 64, C 16, a quarter of the column
    blocks per row block, GQA 32/8, bf16), default workers, sampled rows."""
    w = wl.bsr_sparse()
    say(f"[case] {w.name}")
    o, l = run_bsr(w)
    rng = np.random.Generator(np.random.PCG64(12))
    rows = sorted(set([0, 63, 64, w.M - 1] + list(rng.integers(0, w.M, size=28))))
    o_ref, l_ref = ora.bsr_attention(w.q, w.k, w.v, w.R, w.C, w.indptr, w.indices, "bf16", 8,
                                     rows=rows)
    assert_parity(o, l, o_ref, l_ref, "bf16", rows=rows, what="bsr full sampled")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))


# ----------------------------------------------------------------------------
# page append
# ----------------------------------------------------------------------------
def run_page_append(w):
    import torch
    kv = w.kv
    dev = upload_kv(kv)
    kn = wl.to_torch(w.k_new, kv.dtype, "cuda")
    vn = wl.to_torch(w.v_new, kv.dtype, "cuda")
    abp.append_paged_kv_cache(kn, vn, i32(w.append_indptr), dev["k"], dev["v"], dev["indptr"],
                              dev["indices"], dev["lpl"])
    torch.cuda.synchronize()
    kp = dev["k"].cpu().view(torch.int16).numpy().view(np.uint16)
    vp = dev["v"].cpu().view(torch.int16).numpy().view(np.uint16)
    return kp, vp, dev


@pytest.mark.parametrize("P,hkv,dtype", [(1, 1, "bf16"), (3, 3, "fp16"), (16, 8, "bf16"),
                                         (16, 12, "bf16"), (256, 2, "fp16")])
def test_page_append_bit_exact(P, hkv, dtype):
    say(f"[case] page append P={P} hkv={hkv} {dtype}")
    kv_lens = [0, 5, 1, 300, 17, 64, 1000]
    app = [0, 5, 1, 37, 0, 64, 999]
    w = wl.page_append(500 + P + hkv, kv_lens, app, P, hkv, dtype=dtype)
    kv = w.kv
    kp_ref, vp_ref = ora.append_paged_kv(w.k_new, w.v_new, w.append_indptr, kv.k_pages,
                                         kv.v_pages, kv.kv_indptr, kv.kv_indices,
                                         kv.kv_last_page_len, P)
    kp, vp, _ = run_page_append(w)
    assert np.array_equal(kp, kp_ref) and np.array_equal(vp, vp_ref)


def test_page_append_skips_rows_outside_their_request():
    # request 1 claims 4 new rows but holds 2 tokens: its first 2 rows are skipped
    w = wl.page_append(510, [9, 2, 33], [3, 2, 5], 4, 2)
    pick = [0, 1, 2, 3, 3, 3, 4, 5, 6, 7, 8, 9]          # rows of request 1: 3, 3, 3, 4
    w.k_new, w.v_new = w.k_new[pick], w.v_new[pick]
    w.append_indptr = np.array([0, 3, 7, 12], np.int32)
    kv = w.kv
    kp_ref, vp_ref = ora.append_paged_kv(w.k_new, w.v_new, w.append_indptr, kv.k_pages,
                                         kv.v_pages, kv.kv_indptr, kv.kv_indices,
                                         kv.kv_last_page_len, 4)
    kp, vp, _ = run_page_append(w)
    assert np.array_equal(kp, kp_ref) and np.array_equal(vp, vp_ref)


def test_page_append_full_then_decode():
    """The benchmark's page-append shape (16 requests, 128..1024 new tokens after
    1024..8192 existing, 8 kv heads, page 16, bf16): whole pools bit-exact, then a
    decode over the updated cache against the oracle on the oracle's pools."""
    import torch
    w = wl.ragged_page_append()
    say(f"[case] {w.name}")
    kv = w.kv
    kp_ref, vp_ref = ora.append_paged_kv(w.k_new, w.v_new, w.append_indptr, kv.k_pages,
                                         kv.v_pages, kv.kv_indptr, kv.kv_indices,
                                         kv.kv_last_page_len, 16)
    kp, vp, dev = run_page_append(w)
    assert np.array_equal(kp, kp_ref) and np.array_equal(vp, vp_ref)
    rng = np.random.Generator(np.random.PCG64(13))
    q = wl.normal_bits(rng, (kv.batch, 32, 128), "bf16")
    kv2 = wl.PagedKV(16, 8, 128, "bf16", kv.kv_len, kv.kv_indptr, kv.kv_indices,
                     kv.kv_last_page_len, kp_ref, vp_ref)
    dw = wl.Workload("decode_after_append", "decode", 0, "bf16", 32, 8, 128, kv2, q)
    o, l = run_decode(dw, dev=dev)
    ids = [0, 5, 15]
    o_ref, l_ref = ora.decode_workload(dw, batch_ids=ids)
    assert_parity(o, l, o_ref, l_ref, "bf16", rows=ids, what="decode after page append")


# ----------------------------------------------------------------------------
# LLaMA 3.1 RoPE
# ----------------------------------------------------------------------------
def test_llama31_rope_decode_and_append():
    w = wl.small_decode(600, [1, 40, 3000, 9000], 16, 32, 8)
    w.rope_theta = 500000.0
    w.rope_llama31 = abp.LLAMA31_ROPE
    o_ref, l_ref = ora.decode_workload(w)
    o, l = run_decode(w, num_workers=23)
    assert_parity(o, l, o_ref, l_ref, "bf16", what="llama31 rope decode")
    wa = wl.small_append(601, [3, 90, 200], [50, 400, 9000], 16, 8, 2, causal=True)
    wa.rope_theta = 500000.0
    wa.rope_llama31 = abp.LLAMA31_ROPE
    o_ref, l_ref = ora.append_workload(wa)
    o, l = run_append(wa, num_workers=7)
    assert_parity(o, l, o_ref, l_ref, "bf16", what="llama31 rope append")


# ----------------------------------------------------------------------------
# fp8 (e4m3) KV cache decode
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("P,G,hkv,dtype", [(16, 4, 8, "bf16"), (16, 1, 2, "bf16"),
                                           (3, 4, 2, "fp16"), (16, 8, 4, "fp16"),
                                           (256, 2, 8, "bf16"), (1, 8, 1, "bf16")])
def test_fp8_decode_parity(P, G, hkv, dtype):
    say(f"[case] fp8 decode P={P} G={G} hkv={hkv} q {dtype}")
    w = wl.small_decode_fp8(700 + P + G + hkv, [0, 1, 16, 63, 700, 3000], P, G * hkv, hkv,
                            dtype=dtype, k_scale=0.25, v_scale=0.5)
    o_ref, l_ref = ora.decode_workload(w)
    for W in (1, 29, 0):
        o, l = run_decode(w, num_workers=W)
        assert_parity(o, l, o_ref, l_ref, dtype, what=f"fp8 decode P{P} G{G} hkv{hkv} W{W}")


def test_fp8_decode_stage_tails():
    """fp8 decode segments of 1 to 9 whole 32-token chunks and partial ones, each
    request one unsplit segment (one worker per tile), so the four-stage loop
    runs its prologue, steady part and tail at every length."""
    lens = [32, 64, 96, 128, 160, 192, 224, 256, 288, 31, 33, 225]
    say(f"[case] fp8 decode stage tails {lens}")
    w = wl.small_decode_fp8(777, lens, 16, 4 * 4, 4, k_scale=0.5, v_scale=0.25)
    o_ref, l_ref = ora.decode_workload(w)
    for W in (abp.ABP_WORKERS_PER_TILE, 0):
        o, l = run_decode(w, num_workers=W)
        assert_parity(o, l, o_ref, l_ref, "bf16", what=f"fp8 decode stage tails W{W}")


def test_fp8_batch_decode_full():
    """The fp8 batch decode shape (64 requests, kv U{512..4096}, GQA 32/8, page 16,
    q bf16, e4m3 K/V with scales 0.25) in the default launch, every request."""
    w = wl.batch_decode_fp8()
    say(f"[case] {w.name}")
    o, l = run_decode(w)
    o_ref, l_ref = ora.decode_workload(w)
    assert_parity(o, l, o_ref, l_ref, "bf16", what="fp8 batch decode, all requests")
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(l))


def test_page_append_fp8_bit_exact():
    w = wl.page_append(720, [5, 300, 17, 1000], [5, 37, 1, 999], 16, 8)
    rng = np.random.Generator(np.random.PCG64(721))
    w.kv = wl.to_fp8_kv(rng, w.kv, 0.25)
    w.k_new = wl.round_to_fp8_e4m3(rng.standard_normal(w.k_new.shape, dtype=np.float32) * 4)
    w.v_new = wl.round_to_fp8_e4m3(rng.standard_normal(w.v_new.shape, dtype=np.float32) * 4)
    kv = w.kv
    kp_ref, vp_ref = ora.append_paged_kv(w.k_new, w.v_new, w.append_indptr, kv.k_pages,
                                         kv.v_pages, kv.kv_indptr, kv.kv_indices,
                                         kv.kv_last_page_len, 16)
    import torch
    dev = upload_kv(kv)
    kn = wl.to_torch(w.k_new, "fp8_e4m3", "cuda")
    vn = wl.to_torch(w.v_new, "fp8_e4m3", "cuda")
    abp.append_paged_kv_cache(kn, vn, i32(w.append_indptr), dev["k"], dev["v"], dev["indptr"],
                              dev["indices"], dev["lpl"])
    torch.cuda.synchronize()
    kp = dev["k"].cpu().view(torch.uint8).numpy()
    vp = dev["v"].cpu().view(torch.uint8).numpy()
    assert np.array_equal(kp, kp_ref) and np.array_equal(vp, vp_ref)


# ----------------------------------------------------------------------------
# interleaved (adjacent-pair) RoPE
# ----------------------------------------------------------------------------
@pytest.mark.parametrize("P,G,hkv", [(16, 4, 8), (3, 4, 2), (16, 8, 2), (16, 1, 4)])
def test_interleaved_rope_decode(P, G, hkv):
    w = wl.small_decode(800 + P + G, [1, 40, 700, 3000], P, G * hkv, hkv)
    w.rope_theta = 500000.0
    w.rope_interleave = True
    rng = np.random.Generator(np.random.PCG64(801))
    w.kv_pos_offset = rng.integers(0, 9000, size=w.batch).astype(np.int32)
    w.q_pos = (w.kv_pos_offset + w.kv.kv_len - 1).astype(np.int32)
    o_ref, l_ref = ora.decode_workload(w)
    o, l = run_decode(w, num_workers=19)
    assert_parity(o, l, o_ref, l_ref, "bf16", what=f"interleaved rope decode P{P} G{G}")


@pytest.mark.parametrize("P,causal,l31", [(16, True, False), (3, True, True), (16, False, True)])
def test_interleaved_rope_append(P, causal, l31):
    w = wl.small_append(810 + P, [3, 90, 200], [50, 400, 900], P, 8, 2, causal=causal)
    w.rope_theta = 500000.0
    w.rope_interleave = True
    w.rope_llama31 = abp.LLAMA31_ROPE if l31 else None
    o_ref, l_ref = ora.append_workload(w)
    o, l = run_append(w, num_workers=7)
    assert_parity(o, l, o_ref, l_ref, "bf16", what=f"interleaved rope append P{P} c{int(causal)}")


def test_interleaved_llama31_cascade():
    """Cascade (prefix in pages of 256 + suffixes in pages of 16) with interleaved
    LLaMA 3.1 RoPE: the append (prefix) and decode (suffix) kernels both rotate."""
    import torch
    rng = np.random.Generator(np.random.PCG64(820))
    B, pre_len = 5, 700
    prefix = wl.make_paged_kv(rng, np.array([pre_len]), 256, 2, 128, "bf16", extra_pages=1)
    suf = rng.integers(1, 300, size=B)
    kv = wl.make_paged_kv(rng, suf, 16, 2, 128, "bf16", extra_pages=3)
    q = wl.normal_bits(rng, (B, 8, 128), "bf16")
    w = wl.Workload("small_cascade_il", "cascade", 820, "bf16", 8, 2, 128, kv, q,
                    rope_theta=500000.0, prefix=prefix, rope_llama31=abp.LLAMA31_ROPE,
                    rope_interleave=True)
    w.kv_pos_offset = np.full(B, pre_len, np.int32)
    w.q_pos = (pre_len + suf - 1).astype(np.int32)
    o_ref, l_ref = ora.decode_workload(w)
    cas = abp.CascadeDecode(8, 2, 128, 256, 16, torch.bfloat16, max_batch=B,
                            rope_theta=500000.0, num_workers=9, prefix_workers=4,
                            rope_llama31=abp.LLAMA31_ROPE, rope_interleave=True)
    cas.plan(B, prefix.kv_indptr, prefix.kv_last_page_len, kv.kv_indptr, kv.kv_last_page_len)
    dp, ds = upload_kv(prefix), upload_kv(kv)
    qt = wl.to_torch(q, "bf16", "cuda")
    o, l = cas.run(qt, dp["k"], dp["v"], i32([0, B]), dp["indptr"], dp["indices"], dp["lpl"],
                   ds["k"], ds["v"], ds["indptr"], ds["indices"], ds["lpl"],
                   q_pos=i32(w.q_pos), kv_pos_offset=i32(w.kv_pos_offset))
    torch.cuda.synchronize()
    assert_parity(o.float().cpu().numpy(), l.cpu().numpy(), o_ref, l_ref, "bf16",
                  what="interleaved llama31 cascade")
