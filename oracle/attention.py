"""fp64 CPU oracle for attention over a paged block-sparse-row (BSR) KV cache.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. It shares
no code with the HIP library and imports nothing from it.

What it computes
----------------
The method is exact attention, computed faster (FlashInfer paper summary,
"图谱动态｜学苑周刊 NO.266", section 统一的 KV 缓存存储格式, and the
FlashAttention lineage in "FlashInfer 源码级解读", section FlashAttention 的遗产:
tiling only changes where data sits, not the result). So the oracle is the
definition written out in float64:

    s_t = scale * <q, k_t>          over the visible keys t
    lse = m + ln sum_t exp(s_t - m),  m = max_t s_t   (natural log, scaled logits)
    o   = sum_t exp(s_t - lse) * v_t

with an empty visible set giving o = 0 and lse = -inf. The KV cache of request b
is read by walking its page table in logical order: logical token t lives in
slot ``t % page_size`` of page ``kv_indices[kv_indptr[b] + t // page_size]``,
and only ``kv_last_page_len[b]`` slots of the last page are valid.

Readings of points the pages leave open (each one is listed with its reason in
the design notes):
  * qo head h uses kv head h // (Hq / Hkv) (consecutive qo heads share a kv head);
  * the default scale is 1 / sqrt(head_dim);
  * causal rows are aligned to the end of the KV: query i of a request with
    qo_len queries and kv_len keys sees keys t <= kv_len - qo_len + i;
  * RoPE is LLaMA rotate-half: pairs (j, j + d/2), angle pos * theta^(-2j/d).

Parity pins: brute-force / closed-form / invariant checks live in
``tests/test_oracle_pins.py``; none of them re-types these formulas.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -math.inf


# ----------------------------------------------------------------------------
# storage decoding (exact)
# ----------------------------------------------------------------------------
def fp8_e4m3_to_f64(codes) -> np.ndarray:
    """Exact float64 values of OCP FP8 E4M3 codes (uint8): 1 sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6);
    S.1111.111 is NaN and there is no infinity (largest finite value 448)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & ((c & 0x7) == 7), np.nan, val)
    return sign * val


def storage_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 values of fp16 / bf16 bit patterns (uint16 arrays) or of
    fp8 e4m3 codes (uint8 arrays, dtype "fp8_e4m3")."""
    if dtype == "fp8_e4m3":
        return fp8_e4m3_to_f64(bits)
    b = np.asarray(bits, dtype=np.uint16)
    if dtype == "fp16":
        return b.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# page table walk (BSR addressing)
# ----------------------------------------------------------------------------
def request_kv_len(kv_indptr, kv_last_page_len, page_size: int, b: int) -> int:
    """Number of valid tokens of request b: (n_pages - 1) * page_size + last_page_len."""
    n = int(kv_indptr[b + 1]) - int(kv_indptr[b])
    if n == 0:
        return 0
    return (n - 1) * int(page_size) + int(kv_last_page_len[b])


def walk_pages(pages: np.ndarray, kv_indptr, kv_indices, kv_last_page_len, page_size: int,
               b: int) -> np.ndarray:
    """Logical KV rows of request b, ``[kv_len, Hkv, d]``, gathered page by page.

    ``pages`` is one pool ``[num_pages, page_size, Hkv, d]`` (K or V), in any
    dtype; the rows are returned in that dtype.
    """
    start, end = int(kv_indptr[b]), int(kv_indptr[b + 1])
    kv_len = request_kv_len(kv_indptr, kv_last_page_len, page_size, b)
    out = np.empty((kv_len,) + pages.shape[2:], dtype=pages.dtype)
    t = 0
    for slot in range(start, end):
        page = int(kv_indices[slot])
        take = page_size if slot < end - 1 else int(kv_last_page_len[b])
        out[t:t + take] = pages[page, :take]
        t += take
    assert t == kv_len
    return out


# ----------------------------------------------------------------------------
# RoPE (LLaMA style, rotate-half)
# ----------------------------------------------------------------------------
def rope_inv_freq(head_dim: int, theta: float, llama31=None) -> np.ndarray:
    """theta^(-2j/d) for j in [0, d/2), in float64.

    ``llama31 = (factor, low_freq_factor, high_freq_factor, old_context_len)``
    applies the LLaMA 3.1 frequency scaling (the README page lists LLaMA 3.1
    RoPE among its operators, section 其他算子; the rule is the one published
    with the LLaMA 3.1 models): with wavelength w = 2 pi / f, a frequency whose
    wavelength is shorter than old_context_len / high_freq_factor is kept, one
    whose wavelength is longer than old_context_len / low_freq_factor is divided
    by factor, and in between the two are blended with weight
    s = (old_context_len / w - low_freq_factor) / (high_freq_factor - low_freq_factor)
    on the kept frequency: f' = (1 - s) f / factor + s f.
    """
    j = np.arange(head_dim // 2, dtype=np.float64)
    f = np.power(float(theta), -2.0 * j / head_dim)
    if llama31 is None:
        return f
    factor, low, high, old = (float(x) for x in llama31)
    out = np.empty_like(f)
    for i, fi in enumerate(f):
        w = 2.0 * math.pi / fi
        if w < old / high:
            out[i] = fi
        elif w > old / low:
            out[i] = fi / factor
        else:
            s = (old / w - low) / (high - low)
            out[i] = (1.0 - s) * fi / factor + s * fi
    return out


def rope_rotate(x: np.ndarray, pos, theta: float, llama31=None,
                interleave: bool = False) -> np.ndarray:
    """Rotate the last axis of ``x`` (length d) at position(s) ``pos``.

    Pair j is turned by the angle pos * f_j, f_j = theta^(-2j/d) (optionally
    LLaMA 3.1 scaled, see ``rope_inv_freq``). Pair j is (j, j + d/2)
    (rotate-half) or, with ``interleave``, the adjacent elements (2j, 2j + 1):
        x'_a = x_a cos - x_b sin,   x'_b = x_b cos + x_a sin   for pair (a, b).
    ``pos`` broadcasts against ``x.shape[:-1]``.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    ang = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq(d, theta, llama31)
    c, s = np.cos(ang), np.sin(ang)
    if interleave:
        a, b = x[..., 0::2], x[..., 1::2]
        out = np.empty_like(x)
        out[..., 0::2] = a * c - b * s
        out[..., 1::2] = b * c + a * s
        return out
    lo, hi = x[..., :h], x[..., h:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


# ----------------------------------------------------------------------------
# the attention definition
# ----------------------------------------------------------------------------
def attend(qrows: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
           visible: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of ``qrows [r, d]`` over ``K, V [n, d]`` in float64.

    ``visible[i]`` is the number of leading keys row i may see (default: all n).
    Returns ``o [r, d]`` and the natural-log ``lse [r]`` of the scaled logits.
    """
    qrows = np.asarray(qrows, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    r, d = qrows.shape
    n = K.shape[0]
    if visible is None:
        visible = [n] * r
    o = np.zeros((r, V.shape[1] if V.ndim == 2 else d), dtype=np.float64)
    lse = np.full(r, NEG_INF, dtype=np.float64)
    if n == 0 or r == 0:
        return o, lse
    s = scale * (qrows @ K.T)                                   # [r, n]
    lim = np.asarray(visible, dtype=np.int64)
    s = np.where(np.arange(n)[None, :] < lim[:, None], s, NEG_INF)
    has = lim > 0
    if not has.any():
        return o, lse
    sh = s[has]
    m = sh.max(axis=1, keepdims=True)
    lse_h = m[:, 0] + np.log(np.exp(sh - m).sum(axis=1))
    p = np.exp(sh - lse_h[:, None])
    o[has] = p @ V
    lse[has] = lse_h
    return o, lse


def merge(states: Sequence[Tuple[np.ndarray, np.ndarray]]) -> Tuple[np.ndarray, np.ndarray]:
    """Combine attention states (o_i, lse_i) computed over disjoint key sets.

    With m = max_i lse_i: lse = m + ln sum_i exp(lse_i - m) and
    o = sum_i exp(lse_i - lse) o_i; if every lse_i is -inf the result is
    (0, -inf). Works elementwise over leading axes (o: [..., d], lse: [...]).
    """
    os_ = [np.asarray(o, dtype=np.float64) for o, _ in states]
    ls = [np.asarray(l, dtype=np.float64) for _, l in states]
    L = np.stack(ls)                                  # [k, ...]
    m = L.max(axis=0)
    finite = np.isfinite(m)
    m_safe = np.where(finite, m, 0.0)
    w = np.where(np.isfinite(L), np.exp(L - m_safe), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(finite, m_safe + np.log(np.where(finite, tot, 1.0)), NEG_INF)
    o = np.zeros_like(os_[0])
    for oi, Li in zip(os_, ls):
        wi = np.where(np.isfinite(Li) & finite, np.exp(Li - np.where(finite, lse, 0.0)), 0.0)
        o = o + wi[..., None] * oi
    return o, lse


# ----------------------------------------------------------------------------
# batch entry points (page-table walking)
# ----------------------------------------------------------------------------
def _group(num_qo_heads: int, num_kv_heads: int) -> int:
    if num_qo_heads % num_kv_heads:
        raise ValueError("num_qo_heads must be a multiple of num_kv_heads")
    return num_qo_heads // num_kv_heads


def paged_decode(q, k_pages, v_pages, kv_indptr, kv_indices, kv_last_page_len, page_size: int,
                 dtype: str, num_kv_heads: int, sm_scale: Optional[float] = None,
                 rope_theta: float = 0.0, q_pos=None, kv_pos_offset=None,
                 batch_ids: Optional[Iterable[int]] = None, rope_llama31=None,
                 kv_dtype: Optional[str] = None, k_scale: float = 1.0, v_scale: float = 1.0,
                 rope_interleave: bool = False):
    """Decode attention: one query token per request against its paged KV.

    q ``[B, Hq, d]`` (storage bits); returns float64 ``o [B, Hq, d]``,
    ``lse [B, Hq]``. Rows of requests not in ``batch_ids`` are NaN.
    With RoPE, q of request b sits at ``q_pos[b]`` (default kv_len_b - 1) and
    key t at ``kv_pos_offset[b] + t`` (default offset 0).

    ``kv_dtype`` (default ``dtype``) is the storage of the pages; for
    "fp8_e4m3" the keys are k_scale times their codes' values and the values
    v_scale times theirs (one scale per tensor; the README page names FP8
    attention, section 特性, without a scaling scheme).
    """
    kvd = dtype if kv_dtype is None else kv_dtype
    B, Hq, d = q.shape
    G = _group(Hq, num_kv_heads)
    scale = (1.0 / math.sqrt(d)) if not sm_scale or sm_scale <= 0 else float(sm_scale)
    o = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    for b in (range(B) if batch_ids is None else batch_ids):
        kv_len = request_kv_len(kv_indptr, kv_last_page_len, page_size, b)
        K = float(k_scale) * storage_to_f64(
            walk_pages(k_pages, kv_indptr, kv_indices, kv_last_page_len, page_size, b), kvd)
        V = float(v_scale) * storage_to_f64(
            walk_pages(v_pages, kv_indptr, kv_indices, kv_last_page_len, page_size, b), kvd)
        qb = storage_to_f64(q[b], dtype)
        if rope_theta:
            qp = (kv_len - 1) if q_pos is None else int(q_pos[b])
            off = 0 if kv_pos_offset is None else int(kv_pos_offset[b])
            qb = rope_rotate(qb, qp, rope_theta, rope_llama31, rope_interleave)
            K = rope_rotate(K, (off + np.arange(kv_len))[:, None], rope_theta, rope_llama31,
                            rope_interleave)
        for h in range(num_kv_heads):
            ob, lb = attend(qb[h * G:(h + 1) * G], K[:, h], V[:, h], scale)
            o[b, h * G:(h + 1) * G] = ob
            lse[b, h * G:(h + 1) * G] = lb
    return o, lse


def paged_append(q, qo_indptr, k_pages, v_pages, kv_indptr, kv_indices, kv_last_page_len,
                 page_size: int, dtype: str, num_kv_heads: int, causal: bool = True,
                 sm_scale: Optional[float] = None, rope_theta: float = 0.0, q_pos=None,
                 kv_pos_offset=None, batch_ids: Optional[Iterable[int]] = None,
                 token_ids: Optional[Iterable[int]] = None, rope_llama31=None,
                 rope_interleave: bool = False):
    """Append / prefill attention for ragged queries ``q [sum qo, Hq, d]``.

    Query i (0-based within request b, qo_len_b queries) sees keys
    t <= kv_len_b - qo_len_b + i when ``causal``, else all kv_len_b keys.
    With RoPE, query token j sits at ``q_pos[j]`` (default kv_len_b - qo_len_b + i)
    and key t at ``kv_pos_offset[b] + t``. ``token_ids`` (global query-token
    indices) restricts the rows computed; other rows are NaN.
    """
    T, Hq, d = q.shape
    G = _group(Hq, num_kv_heads)
    scale = (1.0 / math.sqrt(d)) if not sm_scale or sm_scale <= 0 else float(sm_scale)
    B = len(qo_indptr) - 1
    o = np.full((T, Hq, d), np.nan)
    lse = np.full((T, Hq), np.nan)
    want = None if token_ids is None else set(int(t) for t in token_ids)
    for b in (range(B) if batch_ids is None else batch_ids):
        q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
        rows = [j for j in range(q0, q1) if want is None or j in want]
        if not rows:
            continue
        qo_len = q1 - q0
        kv_len = request_kv_len(kv_indptr, kv_last_page_len, page_size, b)
        if causal and qo_len > kv_len:
            raise ValueError("causal append needs qo_len <= kv_len")
        K = storage_to_f64(walk_pages(k_pages, kv_indptr, kv_indices, kv_last_page_len, page_size, b), dtype)
        V = storage_to_f64(walk_pages(v_pages, kv_indptr, kv_indices, kv_last_page_len, page_size, b), dtype)
        Q = storage_to_f64(q[rows], dtype)                     # [r, Hq, d]
        ii = np.asarray(rows) - q0
        if rope_theta:
            qp = (kv_len - qo_len + ii) if q_pos is None else np.asarray(q_pos)[rows]
            off = 0 if kv_pos_offset is None else int(kv_pos_offset[b])
            Q = rope_rotate(Q, np.asarray(qp)[:, None], rope_theta, rope_llama31, rope_interleave)
            K = rope_rotate(K, (off + np.arange(kv_len))[:, None], rope_theta, rope_llama31,
                            rope_interleave)
        vis = (kv_len - qo_len + ii + 1) if causal else np.full(len(rows), kv_len)
        for hq in range(Hq):
            h = hq // G
            ob, lb = attend(Q[:, hq], K[:, h], V[:, h], scale, vis)
            o[rows, hq] = ob
            lse[rows, hq] = lb
    return o, lse


def cascade_decode(q, prefix_k, prefix_v, prefix_indptr, prefix_indices, prefix_last_page_len,
                   prefix_page_size: int, k_pages, v_pages, kv_indptr, kv_indices,
                   kv_last_page_len, page_size: int, dtype: str, num_kv_heads: int,
                   sm_scale: Optional[float] = None, rope_theta: float = 0.0, q_pos=None,
                   kv_pos_offset=None, batch_ids: Optional[Iterable[int]] = None,
                   rope_llama31=None, rope_interleave: bool = False):
    """Decode over a shared prefix (one BSR row in large pages) plus per-request
    suffixes (small pages), combined through their attention states.

    Composable-format reading of the paper summary (section 统一的 KV 缓存存储格式
    and 高级功能): every request attends the whole prefix, whose keys sit at
    positions 0..prefix_len-1, and its own suffix, whose key t sits at
    ``kv_pos_offset[b] + t`` (default prefix_len + t); the query sits at
    ``q_pos[b]`` (default: the last suffix position). The two states are merged
    with ``merge``.
    """
    B = q.shape[0]
    n_pre = int(prefix_indptr[1]) - int(prefix_indptr[0])
    pre_len = request_kv_len(prefix_indptr, prefix_last_page_len, prefix_page_size, 0)
    if kv_pos_offset is None:
        kv_pos_offset = np.full(B, pre_len, dtype=np.int64)
    if q_pos is None:
        q_pos = np.array([int(kv_pos_offset[b])
                          + request_kv_len(kv_indptr, kv_last_page_len, page_size, b) - 1
                          for b in range(B)])
    # prefix level: request b's page list is the shared prefix row
    rep_indptr = np.arange(B + 1, dtype=np.int64) * n_pre
    rep_indices = np.tile(np.asarray(prefix_indices[prefix_indptr[0]:prefix_indptr[1]]), B)
    rep_lpl = np.full(B, int(prefix_last_page_len[0]))
    o_p, l_p = paged_decode(q, prefix_k, prefix_v, rep_indptr, rep_indices, rep_lpl,
                            prefix_page_size, dtype, num_kv_heads, sm_scale, rope_theta,
                            q_pos=q_pos, kv_pos_offset=np.zeros(B, np.int64), batch_ids=batch_ids,
                            rope_llama31=rope_llama31, rope_interleave=rope_interleave)
    # suffix level
    o_s, l_s = paged_decode(q, k_pages, v_pages, kv_indptr, kv_indices, kv_last_page_len,
                            page_size, dtype, num_kv_heads, sm_scale, rope_theta, q_pos=q_pos,
                            kv_pos_offset=kv_pos_offset, batch_ids=batch_ids,
                            rope_llama31=rope_llama31, rope_interleave=rope_interleave)
    ids = list(range(B) if batch_ids is None else batch_ids)
    o = np.full(q.shape, np.nan)
    lse = np.full(q.shape[:2], np.nan)
    o[ids], lse[ids] = merge([(o_p[ids], l_p[ids]), (o_s[ids], l_s[ids])])
    return o, lse


def decode_workload(w, batch_ids=None):
    """Oracle result for a decode or cascade workload object (see the workload generator)."""
    kv = w.kv
    if w.kind == "cascade":
        p = w.prefix
        return cascade_decode(w.q, p.k_pages, p.v_pages, p.kv_indptr, p.kv_indices,
                              p.kv_last_page_len, p.page_size, kv.k_pages, kv.v_pages,
                              kv.kv_indptr, kv.kv_indices, kv.kv_last_page_len, kv.page_size,
                              w.dtype, w.num_kv_heads, w.sm_scale, w.rope_theta, w.q_pos,
                              w.kv_pos_offset, batch_ids, rope_llama31=w.rope_llama31,
                              rope_interleave=w.rope_interleave)
    return paged_decode(w.q, kv.k_pages, kv.v_pages, kv.kv_indptr, kv.kv_indices,
                        kv.kv_last_page_len, kv.page_size, w.dtype, w.num_kv_heads, w.sm_scale,
                        w.rope_theta, w.q_pos, w.kv_pos_offset, batch_ids,
                        rope_llama31=w.rope_llama31, kv_dtype=kv.dtype,
                        k_scale=w.k_scale, v_scale=w.v_scale, rope_interleave=w.rope_interleave)


def append_workload(w, batch_ids=None, token_ids=None):
    """Oracle result for an append workload object (see the workload generator)."""
    kv = w.kv
    return paged_append(w.q, w.qo_indptr, kv.k_pages, kv.v_pages, kv.kv_indptr, kv.kv_indices,
                        kv.kv_last_page_len, kv.page_size, w.dtype, w.num_kv_heads, w.causal,
                        w.sm_scale, w.rope_theta, w.q_pos, w.kv_pos_offset, batch_ids, token_ids,
                        rope_llama31=w.rope_llama31, rope_interleave=w.rope_interleave)


# ----------------------------------------------------------------------------
# block-sparse attention (a BSR mask over a dense K/V)
# ----------------------------------------------------------------------------
def bsr_mask(M: int, N: int, R: int, C: int, indptr, indices) -> np.ndarray:
    """Dense boolean mask ``[M, N]`` of a block-sparse-row pattern.

    Row block i (queries i*R .. min((i+1)*R, M) - 1) lists its column blocks in
    ``indices[indptr[i]:indptr[i+1]]``; column block j covers keys j*C ..
    (j+1)*C - 1. Query r may see key t exactly when the block (r // R, t // C)
    is listed. This is the block-sparse attention of the README page (section
    核心功能, 稀疏注意力机制) on the BSR format of the paper summary (section
    统一的 KV 缓存存储格式).
    """
    mask = np.zeros((M, N), dtype=bool)
    nrb = -(-M // R) if M else 0
    for i in range(nrb):
        r0, r1 = i * R, min((i + 1) * R, M)
        for j in indices[int(indptr[i]):int(indptr[i + 1])]:
            j = int(j)
            mask[r0:r1, j * C:(j + 1) * C] = True
    return mask


def attend_masked(qrows: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                  mask: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of ``qrows [r, d]`` over the keys ``mask[i]`` lets row i
    see (``mask [r, n]`` boolean). A row with no visible key gives o = 0, lse = -inf."""
    qrows = np.asarray(qrows, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    r = qrows.shape[0]
    o = np.zeros((r, V.shape[1]), dtype=np.float64)
    lse = np.full(r, NEG_INF, dtype=np.float64)
    has = mask.any(axis=1)
    if r == 0 or not has.any():
        return o, lse
    s = np.where(mask, scale * (qrows @ K.T), NEG_INF)[has]
    m = s.max(axis=1, keepdims=True)
    lse_h = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
    o[has] = np.exp(s - lse_h[:, None]) @ V
    lse[has] = lse_h
    return o, lse


def bsr_attention(q, k, v, R: int, C: int, indptr, indices, dtype: str, num_kv_heads: int,
                  sm_scale: Optional[float] = None, rows: Optional[Iterable[int]] = None):
    """Block-sparse attention: q ``[M, Hq, d]``, k / v ``[N, Hkv, d]`` (storage
    bits), mask from ``bsr_mask``. Returns float64 ``o [M, Hq, d]``, ``lse [M, Hq]``;
    rows not in ``rows`` (query indices) are NaN."""
    M, Hq, d = q.shape
    N = k.shape[0]
    G = _group(Hq, num_kv_heads)
    scale = (1.0 / math.sqrt(d)) if not sm_scale or sm_scale <= 0 else float(sm_scale)
    ids = np.arange(M) if rows is None else np.asarray(sorted(set(int(r) for r in rows)))
    o = np.full((M, Hq, d), np.nan)
    lse = np.full((M, Hq), np.nan)
    if len(ids) == 0:
        return o, lse
    mask = bsr_mask(M, N, R, C, indptr, indices)[ids]
    K = storage_to_f64(k, dtype)
    V = storage_to_f64(v, dtype)
    Q = storage_to_f64(q[ids], dtype)
    for hq in range(Hq):
        h = hq // G
        ob, lb = attend_masked(Q[:, hq], K[:, h], V[:, h], scale, mask)
        o[ids, hq] = ob
        lse[ids, hq] = lb
    return o, lse


# ----------------------------------------------------------------------------
# appending new tokens to a paged cache
# ----------------------------------------------------------------------------
def append_paged_kv(k_new, v_new, append_indptr, k_pages, v_pages, kv_indptr, kv_indices,
                    kv_last_page_len, page_size: int):
    """Write new K/V rows into copies of the page pools and return them.

    The page table already covers the new tokens (they are the last ones of
    each request): new row i of request b (rows append_indptr[b] ..
    append_indptr[b+1] - 1) is logical token kv_len_b - append_len_b + i, which
    lives in slot (t % page_size) of page kv_indices[kv_indptr[b] + t // page_size].
    This is the step that fills the paged cache before decode / append read it
    (README page, section 核心功能: paged KV caches for dynamic batching).
    Rows whose position would fall outside [0, kv_len_b) are not written.
    """
    kp = np.array(k_pages, copy=True)
    vp = np.array(v_pages, copy=True)
    B = len(append_indptr) - 1
    for b in range(B):
        a0, a1 = int(append_indptr[b]), int(append_indptr[b + 1])
        n = a1 - a0
        kv_len = request_kv_len(kv_indptr, kv_last_page_len, page_size, b)
        for i in range(n):
            t = kv_len - n + i
            if t < 0 or t >= kv_len:
                continue
            page = int(kv_indices[int(kv_indptr[b]) + t // page_size])
            kp[page, t % page_size] = k_new[a0 + i]
            vp[page, t % page_size] = v_new[a0 + i]
    return kp, vp
