"""Seeded synthetic inputs for paged block-sparse-row (BSR) attention.

This module draws request lengths, page pools and N(0, 1) values and rounds them
to the storage type. It holds none of the attention arithmetic. Both the HIP
path (through the binding) and the fp64 oracle are fed from here; neither of
those imports the other.

Storage convention: every fp16 / bf16 tensor is a numpy ``uint16`` array of bit
patterns. ``to_torch`` reinterprets it as the matching torch dtype.

The KV cache of a batch is a block-sparse-row matrix (FlashInfer paper summary,
"图谱动态｜学苑周刊 NO.266", section 统一的 KV 缓存存储格式): request b owns
pages ``kv_indices[kv_indptr[b]:kv_indptr[b+1]]`` in logical order, each page
holds ``page_size`` token slots, and only the first ``kv_last_page_len[b]``
slots of its last page are valid. K and V are separate pools of shape
``[num_pages, page_size, num_kv_heads, head_dim]`` (NHD inside a page).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

BF16 = "bf16"
FP16 = "fp16"


# ----------------------------------------------------------------------------
# rounding fp32 -> storage bits (input generation only)
# ----------------------------------------------------------------------------
def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Finite inputs only (the generators draw N(0, 1)).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def round_to_fp16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (numpy rounds to nearest even)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def round_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return round_to_bf16_bits(x)
    if dtype == FP16:
        return round_to_fp16_bits(x)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def normal_bits(rng: np.random.Generator, shape, dtype: str, chunk: int = 1 << 24) -> np.ndarray:
    """N(0, 1) draws in float32, rounded to ``dtype``; generated in chunks to bound memory."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        out[s:e] = round_bits(rng.standard_normal(e - s, dtype=np.float32), dtype)
    return out.reshape(shape)


def round_to_fp8_e4m3(x: np.ndarray) -> np.ndarray:
    """Round float32 values to OCP FP8 E4M3 codes (uint8), nearest-even, with
    PyTorch's float8_e4m3fn conversion (input generation only; |x| <= 448)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def to_torch(bits: np.ndarray, dtype: str, device=None):
    """Reinterpret uint16 storage bits as a torch fp16 / bf16 tensor, or uint8
    fp8 e4m3 codes as a torch float8_e4m3fn tensor."""
    import torch
    if dtype == "fp8_e4m3":
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.uint8)).view(torch.float8_e4m3fn)
        return t.to(device) if device is not None else t

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.bfloat16 if dtype == BF16 else torch.float16)
    return t.to(device) if device is not None else t


# ----------------------------------------------------------------------------
# paged KV cache
# ----------------------------------------------------------------------------
@dataclass
class PagedKV:
    """One BSR-paged KV cache (a batch of requests sharing one page pool)."""

    page_size: int
    num_kv_heads: int
    head_dim: int
    dtype: str
    kv_len: np.ndarray            # int64 [B], the drawn lengths
    kv_indptr: np.ndarray         # int32 [B+1]
    kv_indices: np.ndarray        # int32 [nnz_pages]
    kv_last_page_len: np.ndarray  # int32 [B]
    k_pages: np.ndarray           # uint16 [num_pages, P, Hkv, d]
    v_pages: np.ndarray           # uint16 [num_pages, P, Hkv, d]

    @property
    def batch(self) -> int:
        return int(self.kv_len.shape[0])

    @property
    def num_pages(self) -> int:
        return int(self.k_pages.shape[0])


def page_table(kv_len: np.ndarray, page_size: int, pool: np.ndarray):
    """indptr / indices / last_page_len for lengths ``kv_len``.

    Pages are handed out to the requests in order from ``pool`` (drawing without
    replacement when ``pool`` is a shuffled permutation). A request with no
    tokens owns no page; its last_page_len is 0 (never read).
    """
    kv_len = np.asarray(kv_len, dtype=np.int64)
    npages = (kv_len + page_size - 1) // page_size
    indptr = np.zeros(len(kv_len) + 1, dtype=np.int64)
    indptr[1:] = np.cumsum(npages)
    if indptr[-1] > len(pool):
        raise ValueError("page pool too small")
    indices = np.asarray(pool[: indptr[-1]], dtype=np.int32)
    lpl = np.where(npages > 0, kv_len - (npages - 1) * page_size, 0)
    return indptr.astype(np.int32), indices, lpl.astype(np.int32)


def make_paged_kv(rng: np.random.Generator, kv_len, page_size: int, num_kv_heads: int,
                  head_dim: int, dtype: str, extra_pages: int = 0, shuffle: bool = True) -> PagedKV:
    """Draw a paged KV cache holding ``kv_len[b]`` tokens for each request.

    The pool holds exactly the pages needed (plus ``extra_pages`` unused ones),
    shuffled with ``rng.permutation`` so logical and physical order differ.
    """
    kv_len = np.asarray(kv_len, dtype=np.int64)
    need = int(((kv_len + page_size - 1) // page_size).sum())
    num_pages = need + int(extra_pages)
    pool = rng.permutation(num_pages) if shuffle else np.arange(num_pages)
    indptr, indices, lpl = page_table(kv_len, page_size, pool)
    shape = (num_pages, page_size, num_kv_heads, head_dim)
    k = normal_bits(rng, shape, dtype)
    v = normal_bits(rng, shape, dtype)
    return PagedKV(page_size, num_kv_heads, head_dim, dtype, kv_len, indptr, indices, lpl, k, v)



# Non-finite bit patterns of each storage type: quiet NaN, -inf and +inf for the
# 16-bit types; e4m3 has no infinity, so its two NaN codes (S.1111.111).
NON_FINITE_BITS = {
    "bf16": (0x7FC0, 0xFF80, 0x7F80),
    "fp16": (0x7E00, 0xFC00, 0x7C00),
    "fp8_e4m3": (0x7F, 0xFF),
}


def poison_unwritten(kv: PagedKV) -> PagedKV:
    """A copy of ``kv`` whose slots that hold no token are non-finite.

    The page table defines only the first ``kv_last_page_len[b]`` slots of a
    request's last page and says nothing of pages no request owns; a cache
    allocated without clearing (or reused) holds arbitrary bits there. This
    fills every such slot, in both pools, with the storage type's NaN / inf
    patterns, cycling through them element by element. The valid slots are
    unchanged, so any correct attention over the table gives the same result.
    """
    k = kv.k_pages.copy()
    v = kv.v_pages.copy()
    pat = NON_FINITE_BITS[kv.dtype]
    dt = k.dtype
    owned = np.zeros(k.shape[0], dtype=bool)
    owned[np.asarray(kv.kv_indices, dtype=np.int64)] = True
    P = kv.page_size
    for b in range(len(kv.kv_indptr) - 1):
        s, e = int(kv.kv_indptr[b]), int(kv.kv_indptr[b + 1])
        if e > s:
            last = int(kv.kv_indices[e - 1])
            lpl = int(kv.kv_last_page_len[b])
            if lpl < P:
                n = k[last, lpl:].size
                fill = np.resize(np.array(pat, dtype=dt), n).reshape(k[last, lpl:].shape)
                k[last, lpl:] = fill
                v[last, lpl:] = fill[..., ::-1]
    free = ~owned
    if free.any():
        n = k[free].size
        fill = np.resize(np.array(pat, dtype=dt), n).reshape(k[free].shape)
        k[free] = fill
        v[free] = fill
    return PagedKV(kv.page_size, kv.num_kv_heads, kv.head_dim, kv.dtype, kv.kv_len,
                   kv.kv_indptr, kv.kv_indices, kv.kv_last_page_len, k, v)

# ----------------------------------------------------------------------------
# the five named workloads
# ----------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    kind: str                      # "decode" | "append" | "cascade"
    seed: int
    dtype: str
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    kv: PagedKV                    # the (suffix) KV cache
    q: np.ndarray                  # uint16 [B, Hq, d] (decode) or [sum qo, Hq, d] (append)
    qo_indptr: Optional[np.ndarray] = None   # int32 [B+1], append only
    causal: bool = False
    rope_theta: float = 0.0        # 0 -> no RoPE
    rope_llama31: Optional[tuple] = None  # (factor, low_freq_factor, high_freq_factor, old_ctx)
    rope_interleave: bool = False  # RoPE pairs (2j, 2j+1) instead of (j, j + d/2)
    k_scale: float = 1.0           # fp8 K/V pages: value = scale * code value
    v_scale: float = 1.0
    q_pos: Optional[np.ndarray] = None       # int32, per query token
    kv_pos_offset: Optional[np.ndarray] = None  # int32 [B]
    prefix: Optional[PagedKV] = None         # cascade: the shared prefix (one "request")
    meta: Dict[str, object] = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return self.kv.batch

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


def single_decode_mha(seed: int = 1001) -> Workload:
    """Single-request decode: 32 qo = 32 kv heads, d 128, fp16, kv_len 2048 in 128
    pages of 16 in random physical order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    Hq = Hkv = 32
    d, P, L = 128, 16, 2048
    kv_len = np.array([L])
    pool = rng.permutation(L // P)
    indptr, indices, lpl = page_table(kv_len, P, pool)
    q = normal_bits(rng, (1, Hq, d), FP16)
    k = normal_bits(rng, (L // P, P, Hkv, d), FP16)
    v = normal_bits(rng, (L // P, P, Hkv, d), FP16)
    kv = PagedKV(P, Hkv, d, FP16, kv_len, indptr, indices, lpl, k, v)
    return Workload("single_decode_mha32_d128_fp16_kv2048_p16", "decode", seed, FP16, Hq, Hkv, d, kv, q)


def batch_decode_gqa(seed: int = 1002, batch: int = 64, lo: int = 512, hi: int = 4096,
                     num_qo_heads: int = 32) -> Workload:
    """Batch paged decode: 64 requests, GQA 32/8, d 128, page 16, bf16,
    kv_len uniform on the integers [512, 4096] (``num_qo_heads`` = 64 gives
    groups of 8 over the same cache)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    Hq, Hkv, d, P = num_qo_heads, 8, 128, 16
    kv_len = rng.integers(lo, hi, size=batch, endpoint=True)
    q = normal_bits(rng, (batch, Hq, d), BF16)
    kv = make_paged_kv(rng, kv_len, P, Hkv, d, BF16)
    return Workload(f"batch_decode_b{batch}_gqa{Hq}x8_d128_bf16_p16_kv{lo}-{hi}", "decode", seed,
                    BF16, Hq, Hkv, d, kv, q)


def skewed_decode_gqa(seed: int = 1003, batch: int = 128) -> Workload:
    """Skewed-length decode: 128 requests, GQA 32/8, d 128, page 16, bf16; one
    request of 32768 tokens, the rest lognormal(ln 512, 1) rounded and clipped
    to [16, 16384]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    Hq, Hkv, d, P = 32, 8, 128, 16
    rest = np.clip(np.rint(np.exp(rng.normal(np.log(512.0), 1.0, size=batch - 1))), 16, 16384)
    kv_len = np.concatenate([[32768], rest]).astype(np.int64)
    q = normal_bits(rng, (batch, Hq, d), BF16)
    kv = make_paged_kv(rng, kv_len, P, Hkv, d, BF16)
    return Workload(f"skewed_decode_b{batch}_gqa32x8_d128_bf16_p16_long32768", "decode", seed,
                    BF16, Hq, Hkv, d, kv, q)


def ragged_append_causal(seed: int = 1004, batch: int = 16) -> Workload:
    """Ragged causal append: 16 requests each appending qo_len ~ U{128..1024} new
    tokens onto an existing kv_len ~ U{1024..8192}; the page table holds
    existing + qo_len tokens (the new K/V are already cached); GQA 32/8, d 128,
    page 16, bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    Hq, Hkv, d, P = 32, 8, 128, 16
    qo_len = rng.integers(128, 1024, size=batch, endpoint=True)
    existing = rng.integers(1024, 8192, size=batch, endpoint=True)
    kv_len = existing + qo_len
    qo_indptr = np.zeros(batch + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(qo_len)
    q = normal_bits(rng, (int(qo_indptr[-1]), Hq, d), BF16)
    kv = make_paged_kv(rng, kv_len, P, Hkv, d, BF16)
    w = Workload(f"ragged_append_causal_{batch}req_gqa32x8_d128_bf16_p16", "append", seed, BF16,
                 Hq, Hkv, d, kv, q, qo_indptr=qo_indptr, causal=True)
    w.meta["existing"] = existing
    return w


def cascade_rope(seed: int = 1005, batch: int = 64, prefix_len: int = 8192) -> Workload:
    """Cascade (composable formats) decode with fused RoPE: 64 decode requests
    sharing one 8192-token prefix stored in pages of 256, plus unique suffixes of
    U{256..1024} tokens in pages of 16; GQA 32/8, d 128, bf16; LLaMA RoPE with
    theta 500000 on q and k from per-token positions (prefix token t at t,
    suffix token t at prefix_len + t, the query at the last suffix position)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    Hq, Hkv, d = 32, 8, 128
    prefix = make_paged_kv(rng, np.array([prefix_len]), 256, Hkv, d, BF16)
    suffix_len = rng.integers(256, 1024, size=batch, endpoint=True)
    kv = make_paged_kv(rng, suffix_len, 16, Hkv, d, BF16)
    q = normal_bits(rng, (batch, Hq, d), BF16)
    q_pos = (prefix_len + suffix_len - 1).astype(np.int32)
    kv_pos_offset = np.full(batch, prefix_len, dtype=np.int32)
    return Workload(f"cascade_rope_{batch}req_prefix{prefix_len}p256_suffix256-1024p16_gqa32x8_bf16",
                    "cascade", seed, BF16, Hq, Hkv, d, kv, q, rope_theta=500000.0,
                    q_pos=q_pos, kv_pos_offset=kv_pos_offset, prefix=prefix)


WORKLOADS = {
    "single_decode": single_decode_mha,
    "batch_decode": batch_decode_gqa,
    "skewed_decode": skewed_decode_gqa,
    "ragged_append": ragged_append_causal,
    "cascade_rope": cascade_rope,
}


def small_decode(seed: int, kv_lens: List[int], page_size: int, num_qo_heads: int, num_kv_heads: int,
                 head_dim: int = 128, dtype: str = BF16, extra_pages: int = 3) -> Workload:
    """A small decode batch for parity tests (arbitrary lengths, including 0)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    kv = make_paged_kv(rng, np.asarray(kv_lens), page_size, num_kv_heads, head_dim, dtype,
                       extra_pages=extra_pages)
    q = normal_bits(rng, (len(kv_lens), num_qo_heads, head_dim), dtype)
    return Workload(f"small_decode_s{seed}", "decode", seed, dtype, num_qo_heads, num_kv_heads,
                    head_dim, kv, q)


def small_append(seed: int, qo_lens: List[int], kv_lens: List[int], page_size: int,
                 num_qo_heads: int, num_kv_heads: int, head_dim: int = 128, dtype: str = BF16,
                 causal: bool = True, extra_pages: int = 3) -> Workload:
    """A small ragged append batch for parity tests."""
    rng = np.random.Generator(np.random.PCG64(seed))
    kv = make_paged_kv(rng, np.asarray(kv_lens), page_size, num_kv_heads, head_dim, dtype,
                       extra_pages=extra_pages)
    qo_indptr = np.zeros(len(qo_lens) + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(qo_lens)
    q = normal_bits(rng, (int(qo_indptr[-1]), num_qo_heads, head_dim), dtype)
    return Workload(f"small_append_s{seed}", "append", seed, dtype, num_qo_heads, num_kv_heads,
                    head_dim, kv, q, qo_indptr=qo_indptr, causal=causal)


# ----------------------------------------------------------------------------
# block-sparse attention over a dense K/V
# ----------------------------------------------------------------------------
@dataclass
class BsrWorkload:
    """q [M, Hq, d], k / v [N, Hkv, d] (storage bits) and a block-sparse-row mask:
    row block i (R queries) sees column blocks indices[indptr[i]:indptr[i+1]] (C keys each)."""

    name: str
    seed: int
    dtype: str
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    R: int
    C: int
    indptr: np.ndarray    # int32 [ceil(M / R) + 1]
    indices: np.ndarray   # int32 [nnz blocks]
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray

    @property
    def M(self) -> int:
        return int(self.q.shape[0])

    @property
    def N(self) -> int:
        return int(self.k.shape[0])

    @property
    def sm_scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


def bsr_pattern(rng: np.random.Generator, num_row_blocks: int, num_col_blocks: int,
                density: float, empty_rows=()):
    """Each row block lists round(density * num_col_blocks) (at least 1) distinct
    column blocks drawn uniformly without replacement, sorted; rows in
    ``empty_rows`` list none."""
    k = max(1, int(round(density * num_col_blocks)))
    indptr = np.zeros(num_row_blocks + 1, dtype=np.int32)
    rows = []
    for i in range(num_row_blocks):
        if i in empty_rows or num_col_blocks == 0:
            cols = np.zeros(0, dtype=np.int32)
        else:
            cols = np.sort(rng.choice(num_col_blocks, size=min(k, num_col_blocks), replace=False))
        rows.append(cols.astype(np.int32))
        indptr[i + 1] = indptr[i] + len(cols)
    indices = np.concatenate(rows) if rows else np.zeros(0, np.int32)
    return indptr, indices.astype(np.int32)


def small_bsr(seed: int, M: int, N: int, R: int, C: int, num_qo_heads: int, num_kv_heads: int,
              density: float = 0.3, dtype: str = BF16, head_dim: int = 128,
              empty_rows=()) -> BsrWorkload:
    rng = np.random.Generator(np.random.PCG64(seed))
    nrb = -(-M // R) if M else 0
    indptr, indices = bsr_pattern(rng, nrb, N // C, density, empty_rows)
    q = normal_bits(rng, (M, num_qo_heads, head_dim), dtype)
    k = normal_bits(rng, (N, num_kv_heads, head_dim), dtype)
    v = normal_bits(rng, (N, num_kv_heads, head_dim), dtype)
    return BsrWorkload(f"small_bsr_s{seed}", seed, dtype, num_qo_heads, num_kv_heads, head_dim,
                       R, C, indptr, indices, q, k, v)


def bsr_sparse(seed: int = 1006, M: int = 8192, N: int = 8192, R: int = 64, C: int = 16,
               density: float = 0.25) -> BsrWorkload:
    """Block-sparse attention: one 8192-token sequence, GQA 32/8, d 128, bf16;
    row blocks of 64 queries, column blocks of 16 keys, each row block seeing a
    random quarter of the column blocks."""
    rng = np.random.Generator(np.random.PCG64(seed))
    Hq, Hkv, d = 32, 8, 128
    indptr, indices = bsr_pattern(rng, M // R, N // C, density)
    q = normal_bits(rng, (M, Hq, d), BF16)
    k = normal_bits(rng, (N, Hkv, d), BF16)
    v = normal_bits(rng, (N, Hkv, d), BF16)
    return BsrWorkload(f"bsr_M{M}_N{N}_R{R}_C{C}_density{density}_gqa32x8_d128_bf16", seed,
                       BF16, Hq, Hkv, d, R, C, indptr, indices, q, k, v)


# ----------------------------------------------------------------------------
# new tokens for a paged cache
# ----------------------------------------------------------------------------
@dataclass
class PageAppendWorkload:
    """New K/V rows ``[nnz, Hkv, d]`` ragged by ``append_indptr`` and the paged
    cache (page table already extended to hold them) they are written into."""

    name: str
    seed: int
    kv: PagedKV
    append_indptr: np.ndarray   # int32 [B + 1]
    k_new: np.ndarray
    v_new: np.ndarray

    @property
    def nnz(self) -> int:
        return int(self.append_indptr[-1])


def page_append(seed: int, kv_lens, append_lens, page_size: int, num_kv_heads: int,
                head_dim: int = 128, dtype: str = BF16, extra_pages: int = 2,
                name: str = "") -> PageAppendWorkload:
    """A paged cache of ``kv_lens`` tokens (the last ``append_lens[b]`` of each
    request are the new ones) and the new rows to write."""
    rng = np.random.Generator(np.random.PCG64(seed))
    kv = make_paged_kv(rng, np.asarray(kv_lens), page_size, num_kv_heads, head_dim, dtype,
                       extra_pages=extra_pages)
    ai = np.zeros(len(append_lens) + 1, dtype=np.int32)
    ai[1:] = np.cumsum(append_lens)
    k_new = normal_bits(rng, (int(ai[-1]), num_kv_heads, head_dim), dtype)
    v_new = normal_bits(rng, (int(ai[-1]), num_kv_heads, head_dim), dtype)
    return PageAppendWorkload(name or f"page_append_s{seed}", seed, kv, ai, k_new, v_new)


def ragged_page_append(seed: int = 1007, batch: int = 16) -> PageAppendWorkload:
    """The new tokens of the ragged append shape: 16 requests, qo_len ~ U{128..1024}
    new tokens after an existing kv_len ~ U{1024..8192}; GQA 32/8 (8 kv heads),
    d 128, page 16, bf16."""
    rng = np.random.Generator(np.random.PCG64(seed))
    qo_len = rng.integers(128, 1024, size=batch, endpoint=True)
    existing = rng.integers(1024, 8192, size=batch, endpoint=True)
    return page_append(seed + 1, existing + qo_len, qo_len, 16, 8,
                       name=f"page_append_{batch}req_new128-1024_kv1024-8192_hkv8_d128_bf16_p16")


WORKLOADS_NEXT = {
    "bsr_sparse": bsr_sparse,
    "page_append": ragged_page_append,
}


# ----------------------------------------------------------------------------
# fp8 (e4m3) KV pages
# ----------------------------------------------------------------------------
FP8 = "fp8_e4m3"


def to_fp8_kv(rng: np.random.Generator, kv: PagedKV, scale: float) -> PagedKV:
    """The same page table with fresh N(0, 1) K/V stored as e4m3 codes of
    value / scale (so value ~ scale * code)."""
    shape = kv.k_pages.shape
    k = round_to_fp8_e4m3(rng.standard_normal(shape, dtype=np.float32) / np.float32(scale))
    v = round_to_fp8_e4m3(rng.standard_normal(shape, dtype=np.float32) / np.float32(scale))
    return PagedKV(kv.page_size, kv.num_kv_heads, kv.head_dim, FP8, kv.kv_len, kv.kv_indptr,
                   kv.kv_indices, kv.kv_last_page_len, k, v)


def small_decode_fp8(seed: int, kv_lens, page_size: int, num_qo_heads: int, num_kv_heads: int,
                     dtype: str = BF16, k_scale: float = 0.25, v_scale: float = 0.5) -> Workload:
    """A small decode batch whose K/V pages hold e4m3 codes (q in ``dtype``)."""
    w = small_decode(seed, kv_lens, page_size, num_qo_heads, num_kv_heads, dtype=dtype)
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    w.kv = to_fp8_kv(rng, w.kv, 1.0)
    w.k_scale, w.v_scale = float(k_scale), float(v_scale)
    w.name = f"small_decode_fp8_s{seed}"
    return w


def batch_decode_fp8(seed: int = 1009) -> Workload:
    """Batch paged decode with an fp8 KV cache: the batch decode shape (64
    requests, kv_len U{512..4096}, GQA 32/8, d 128, page 16), q bf16, K/V e4m3
    codes of N(0, 1) / 0.25 with k_scale = v_scale = 0.25."""
    w = batch_decode_gqa(seed)
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    w.kv = to_fp8_kv(rng, w.kv, 0.25)
    w.k_scale = w.v_scale = 0.25
    w.name = "batch_decode_fp8kv_b64_gqa32x8_d128_p16_kv512-4096"
    return w


# ----------------------------------------------------------------------------
# mixed batches: decode and append requests over one page pool
# ----------------------------------------------------------------------------
@dataclass
class PodWorkload:
    """Decode requests and append requests of one KV cache: both parts' page
    tables index the same pools (k_pages, v_pages)."""
    name: str
    dec: Workload                 # kv.k_pages / kv.v_pages are the shared pools
    app: Workload                 # its kv_indices index the shared pools too
    meta: Dict[str, object] = field(default_factory=dict)


def mixed_batch(dec: Workload, app: Workload, name: str) -> PodWorkload:
    """Put the pages of an append workload after those of a decode workload in
    one pool and shift the append page table accordingly."""
    assert dec.kv.page_size == app.kv.page_size and dec.dtype == app.dtype
    n = dec.kv.k_pages.shape[0]
    k = np.concatenate([dec.kv.k_pages, app.kv.k_pages])
    v = np.concatenate([dec.kv.v_pages, app.kv.v_pages])
    dkv = PagedKV(dec.kv.page_size, dec.kv.num_kv_heads, dec.kv.head_dim, dec.kv.dtype,
                  dec.kv.kv_len, dec.kv.kv_indptr, dec.kv.kv_indices, dec.kv.kv_last_page_len,
                  k, v)
    akv = PagedKV(app.kv.page_size, app.kv.num_kv_heads, app.kv.head_dim, app.kv.dtype,
                  app.kv.kv_len, app.kv.kv_indptr, (app.kv.kv_indices + n).astype(np.int32),
                  app.kv.kv_last_page_len, k, v)
    dec.kv, app.kv = dkv, akv
    return PodWorkload(name, dec, app)


def pod_mixed(seed: int = 1010) -> PodWorkload:
    """A mixed batch: the batch decode shape (64 requests, kv_len U{512..4096},
    GQA 32/8, d 128, page 16, bf16; seed 1010) beside a chunked prefill of 4
    requests, each appending a 512-token chunk causally onto existing kv_len
    U{1024..4096} (seed 1011), in one page pool."""
    dec = batch_decode_gqa(seed)
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    Hq, Hkv, d, P, B = 32, 8, 128, 16, 4
    qo_len = np.full(B, 512)
    existing = rng.integers(1024, 4096, size=B, endpoint=True)
    qo_indptr = np.zeros(B + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(qo_len)
    q = normal_bits(rng, (int(qo_indptr[-1]), Hq, d), BF16)
    kv = make_paged_kv(rng, existing + qo_len, P, Hkv, d, BF16)
    app = Workload("chunked_prefill_4x512", "append", seed + 1, BF16, Hq, Hkv, d, kv, q,
                   qo_indptr=qo_indptr, causal=True)
    return mixed_batch(dec, app, "pod_decode64_kv512-4096_prefill4x512_gqa32x8_d128_bf16_p16")
