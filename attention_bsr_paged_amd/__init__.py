"""attention_bsr_paged_amd: paged block-sparse-row attention for AMD MI355X (gfx950).

Python binding of ``libabp.so`` (C ABI declared in ``include/abp.h``). The
``abp_*`` functions keep the C names and only marshal arguments; the helper
classes take torch tensors (torch is used for device memory and streams only)
and call the same entry points. Every step of the computation runs in the HIP
kernels of the library: if ``libabp.so`` is missing, loading raises.

Typical decode step::

    params = make_params(32, 8, 128, page_size=16, dtype=torch.bfloat16)
    dec = BatchDecode(params, max_batch=64)
    dec.plan(kv_indptr_cpu, kv_last_page_len_cpu)          # CPU planner + upload
    o, lse = dec.run(q, k_pages, v_pages, kv_indptr, kv_indices, kv_last_page_len)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

__all__ = [
    "ABP_OK", "ABP_ERR_INVALID_ARG", "ABP_ERR_UNSUPPORTED", "ABP_ERR_WORKSPACE_TOO_SMALL",
    "ABP_ERR_PLAN_MISMATCH", "ABP_ERR_HIP", "ABP_F16", "ABP_BF16", "ABP_F32",
    "ABP_KIND_DECODE", "ABP_KIND_APPEND", "ABP_KIND_BSR", "AbpParams", "AbpPlan", "AbpError",
    "load_library", "library_path", "make_params", "BatchDecode", "BatchAppend", "merge_state",
    "merge_states", "single_decode_with_kv_cache", "CascadeDecode", "BlockSparseAttention",
    "append_paged_kv_cache", "LLAMA31_ROPE", "EXPORTED_SYMBOLS", "AbpPodPlan", "PodAttention",
]

ABP_OK = 0
ABP_ERR_INVALID_ARG = -1
ABP_ERR_UNSUPPORTED = -2
ABP_ERR_WORKSPACE_TOO_SMALL = -3
ABP_ERR_PLAN_MISMATCH = -4
ABP_ERR_HIP = -5

ABP_F16, ABP_BF16, ABP_F32 = 0, 1, 2
ABP_WORKERS_PER_TILE = -1   # num_workers: one worker per tile, no split (ablation)
ABP_KIND_DECODE, ABP_KIND_APPEND, ABP_KIND_BSR = 0, 1, 2

# LLaMA 3.1 RoPE frequency scaling: (factor, low_freq_factor, high_freq_factor,
# old_context_len) as published with those models
LLAMA31_ROPE = (8.0, 1.0, 4.0, 8192.0)

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.environ.get("ABP_LIBRARY", os.path.join(_HERE, "lib", "libabp.so"))


class AbpParams(ctypes.Structure):
    _fields_ = [
        ("num_qo_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("qkv_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("sm_scale", ctypes.c_float),
        ("causal", ctypes.c_int32),
        ("rope", ctypes.c_int32),
        ("rope_theta", ctypes.c_float),
        ("rope_factor", ctypes.c_float),
        ("rope_low_freq_factor", ctypes.c_float),
        ("rope_high_freq_factor", ctypes.c_float),
        ("rope_old_context_len", ctypes.c_float),
        ("kv_fp8", ctypes.c_int32),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
        ("rope_interleave", ctypes.c_int32),
    ]


class AbpPlan(ctypes.Structure):
    _fields_ = [
        ("kind", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("num_workers", ctypes.c_int32),
        ("tile_q", ctypes.c_int32),
        ("tile_kv", ctypes.c_int32),
        ("rows_per_tile", ctypes.c_int32),
        ("num_tiles", ctypes.c_int32),
        ("num_segments", ctypes.c_int32),
        ("num_partials", ctypes.c_int32),
        ("num_merges", ctypes.c_int32),
        ("max_tiles", ctypes.c_int32),
        ("max_segments", ctypes.c_int32),
        ("max_partials", ctypes.c_int32),
        ("upload_path", ctypes.c_int32),
        ("fingerprint", ctypes.c_uint64),
        ("plan_bytes", ctypes.c_uint64),
        ("partial_offset", ctypes.c_uint64),
        ("dev_bytes", ctypes.c_uint64),
    ]


class AbpPodPlan(ctypes.Structure):
    _fields_ = [
        ("decode", AbpPlan),
        ("append", AbpPlan),
        ("num_groups", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("decode_host_offset", ctypes.c_uint64),
        ("append_host_offset", ctypes.c_uint64),
        ("decode_dev_offset", ctypes.c_uint64),
        ("append_dev_offset", ctypes.c_uint64),
        ("decode_dev_bytes", ctypes.c_uint64),
        ("append_dev_bytes", ctypes.c_uint64),
    ]


class AbpError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"abp status {status}: {message}")
        self.status = status
        self.message = message


_i32p = ctypes.POINTER(ctypes.c_int32)
_f32p = ctypes.POINTER(ctypes.c_float)
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_szp = ctypes.POINTER(ctypes.c_size_t)
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_int = ctypes.c_int
_pp = ctypes.POINTER(AbpParams)
_planp = ctypes.POINTER(AbpPlan)
_podp = ctypes.POINTER(AbpPodPlan)

# name -> (restype, argtypes); the order and types follow include/abp.h
_SIGNATURES = {
    "abp_status_string": (ctypes.c_char_p, [_int]),
    "abp_last_error": (ctypes.c_char_p, []),
    "abp_device_num_cus": (_int, [_int, _i32p]),
    "abp_workspace_size": (_int, [_int, _pp, _i32, _i32, _i32, _szp, _szp]),
    "abp_plan_host": (_int, [_int, _pp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _sz, _planp]),
    "abp_decode_plan": (_int, [_pp, _i32, _vp, _vp, _i32, _i32, _vp, _sz, _vp, _sz, _vp, _planp]),
    "abp_decode_run": (_int, [_planp, _pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                              _vp, _sz, _vp]),
    "abp_append_plan": (_int, [_pp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _vp, _sz, _vp, _sz,
                               _vp, _planp]),
    "abp_append_run": (_int, [_planp, _pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                              _vp, _vp, _sz, _vp]),
    "abp_bsr_plan_host": (_int, [_pp, _i32, _i32, _i32, _vp, _i32, _i32, _i32, _vp, _sz, _planp]),
    "abp_bsr_plan": (_int, [_pp, _i32, _i32, _i32, _vp, _i32, _i32, _i32, _vp, _sz, _vp, _sz, _vp,
                            _planp]),
    "abp_bsr_run": (_int, [_planp, _pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "abp_append_paged_kv": (_int, [_pp, _i32, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "abp_pod_workspace_size": (_int, [_pp, _i32, _i32, _i32, _i32, _szp, _szp]),
    "abp_pod_plan_host": (_int, [_pp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32,
                                 _i32, _i32, _vp, _sz, _podp]),
    "abp_pod_plan": (_int, [_pp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                            _i32, _vp, _sz, _vp, _sz, _vp, _podp]),
    "abp_pod_run": (_int, [_podp, _pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                           _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "abp_cascade_run": (_int, [_planp, _pp, _vp, _sz, _planp, _pp, _vp, _sz, _vp, _vp, _vp, _vp,
                               _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                               _vp, _vp, _vp, _i32, _vp]),
    "abp_merge_state": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i32, _int, _int, _vp]),
    "abp_merge_states": (_int, [_vp, _vp, _i32, _i64, _i32, _int, _int, _vp, _vp, _vp]),
    "abp_decode_static": (_int, [_pp, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                 _vp, _vp, _vp, _vp]),
}
ABP_STATIC_SCRATCH_BYTES = 32 << 20
ABP_STATIC_PLAN_BYTES = 1 << 20
EXPORTED_SYMBOLS = tuple(_SIGNATURES)

_lib = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libabp.so (built by ``python -m attention_bsr_paged_amd.build``)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path()
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with `python -m attention_bsr_paged_amd.build`"
                           " (the HIP library is required; there is no fallback)")
    lib = ctypes.CDLL(p)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _check(status: int) -> None:
    if status != ABP_OK:
        lib = load_library()
        raise AbpError(status, lib.abp_last_error().decode(errors="replace"))


# ----------------------------------------------------------------------------
# raw C entry points (same names; pointers are ints or ctypes objects)
# ----------------------------------------------------------------------------
def abp_status_string(status: int) -> str:
    return load_library().abp_status_string(status).decode()


def abp_last_error() -> str:
    return load_library().abp_last_error().decode(errors="replace")


def abp_device_num_cus(device: int = 0) -> int:
    n = ctypes.c_int32()
    _check(load_library().abp_device_num_cus(device, ctypes.byref(n)))
    return n.value


def abp_workspace_size(kind: int, params: AbpParams, max_batch: int, max_qo_tokens: int,
                       num_workers: int):
    h, d = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load_library().abp_workspace_size(kind, ctypes.byref(params), max_batch, max_qo_tokens,
                                             num_workers, ctypes.byref(h), ctypes.byref(d)))
    return h.value, d.value


def abp_plan_host(kind: int, params: AbpParams, batch: int, qo_indptr, kv_indptr,
                  kv_last_page_len, max_batch: int, max_qo_tokens: int, num_workers: int,
                  host_ws: np.ndarray) -> AbpPlan:
    """Host-only planner into a numpy buffer (for inspection and tests)."""
    plan = AbpPlan()
    arrs = [None if a is None else np.ascontiguousarray(a, dtype=np.int32)
            for a in (qo_indptr, kv_indptr, kv_last_page_len)]
    ptrs = [None if a is None else a.ctypes.data for a in arrs]
    _check(load_library().abp_plan_host(kind, ctypes.byref(params), batch, ptrs[0], ptrs[1],
                                        ptrs[2], max_batch, max_qo_tokens, num_workers,
                                        host_ws.ctypes.data, host_ws.nbytes, ctypes.byref(plan)))
    return plan


def abp_bsr_plan_host(params: AbpParams, M: int, N: int, R: int, indptr, max_row_blocks: int,
                      max_M: int, num_workers: int, host_ws: np.ndarray) -> AbpPlan:
    """Host-only block-sparse planner into a numpy buffer (for inspection and tests)."""
    plan = AbpPlan()
    ip = np.ascontiguousarray(indptr, dtype=np.int32)
    _check(load_library().abp_bsr_plan_host(ctypes.byref(params), M, N, R, ip.ctypes.data,
                                            max_row_blocks, max_M, num_workers,
                                            host_ws.ctypes.data, host_ws.nbytes,
                                            ctypes.byref(plan)))
    return plan


def abp_pod_workspace_size(params: AbpParams, max_decode_batch: int, max_append_batch: int,
                           max_qo_tokens: int, num_groups: int):
    h, d = ctypes.c_size_t(), ctypes.c_size_t()
    _check(load_library().abp_pod_workspace_size(ctypes.byref(params), max_decode_batch,
                                                 max_append_batch, max_qo_tokens, num_groups,
                                                 ctypes.byref(h), ctypes.byref(d)))
    return h.value, d.value


def _pod_arrays(d_kv_indptr, d_kv_last_page_len, qo_indptr, a_kv_indptr, a_kv_last_page_len):
    arrs = [np.zeros(1, np.int32) if a is None else _i32_host(a)
            for a in (d_kv_indptr, d_kv_last_page_len, qo_indptr, a_kv_indptr,
                      a_kv_last_page_len)]
    return arrs, len(arrs[0]) - 1, len(arrs[3]) - 1


def abp_pod_plan_host(params: AbpParams, d_kv_indptr, d_kv_last_page_len, qo_indptr,
                      a_kv_indptr, a_kv_last_page_len, max_decode_batch: int,
                      max_append_batch: int, max_qo_tokens: int, num_groups: int,
                      decode_groups: int, host_ws: np.ndarray) -> AbpPodPlan:
    """Host-only mixed-batch planner into a numpy buffer (for inspection and tests)."""
    plan = AbpPodPlan()
    arrs, nd, na = _pod_arrays(d_kv_indptr, d_kv_last_page_len, qo_indptr, a_kv_indptr,
                               a_kv_last_page_len)
    _check(load_library().abp_pod_plan_host(
        ctypes.byref(params), nd, arrs[0].ctypes.data, arrs[1].ctypes.data, na,
        arrs[2].ctypes.data, arrs[3].ctypes.data, arrs[4].ctypes.data, max_decode_batch,
        max_append_batch, max_qo_tokens, num_groups, decode_groups, host_ws.ctypes.data,
        host_ws.nbytes, ctypes.byref(plan)))
    return plan


def decode_plan_arrays(blob: np.ndarray, plan: AbpPlan):
    """Read the plan arrays back out of a plan blob (int32 view), for inspection."""
    b = blob.view(np.int32)
    H = {k: i for i, k in enumerate(
        ["MAGIC", "KIND", "BATCH", "WORKERS", "NUM_TILES", "NUM_SEGS", "NUM_PARTIALS",
         "NUM_MERGES", "TILE_Q", "TILE_KV", "ROWS", "GROUP", "NUM_KV_HEADS", "PAGE_SIZE",
         "NUM_BLOCKS", "QUOTA", "OFF_WSEG", "OFF_SEG", "OFF_TILE", "OFF_MERGE", "OFF_ROPE",
         "MAX_TILES", "MAX_SEGS", "MAX_PARTIALS", "CAUSAL", "OFF_CNT", "OFF_NTILE",
         "MERGE_KERNEL", "TILE_HEADS", "OFF_AUX"])}
    W, T, S, M = b[H["WORKERS"]], b[H["NUM_TILES"]], b[H["NUM_SEGS"]], b[H["NUM_MERGES"]]
    seg = b[b[H["OFF_SEG"]]: b[H["OFF_SEG"]] + 4 * S].reshape(S, 4)
    tile = b[b[H["OFF_TILE"]]: b[H["OFF_TILE"]] + 4 * T].reshape(T, 4)
    mrg = b[b[H["OFF_MERGE"]]: b[H["OFF_MERGE"]] + 4 * M].reshape(M, 4)
    num_partials = b[b[H["OFF_NTILE"]]: b[H["OFF_NTILE"]] + T].copy()
    return {
        "num_blocks": b[H["NUM_BLOCKS"]: H["NUM_BLOCKS"] + 1].copy(),
        "quota": b[H["QUOTA"]: H["QUOTA"] + 1].copy(),
        "num_partials": b[H["NUM_PARTIALS"]: H["NUM_PARTIALS"] + 1].copy(),
        "worker_seg_indptr": b[b[H["OFF_WSEG"]]: b[H["OFF_WSEG"]] + W + 1].copy(),
        "seg_tile": seg[:, 0].copy(), "seg_kv_begin": seg[:, 1].copy(),
        "seg_kv_end": seg[:, 2].copy(), "seg_partial": seg[:, 3].copy(),
        "tile_b": tile[:, 0].copy(), "tile_h": tile[:, 1].copy(), "tile_qt": tile[:, 2].copy(),
        "tile_first_partial": tile[:, 3].copy(), "tile_num_partials": num_partials,
        "merge_list": mrg[:, 0].copy(),
        "merge_kernel": b[H["MERGE_KERNEL"]: H["MERGE_KERNEL"] + 1].copy(),
        "tile_heads": b[H["TILE_HEADS"]: H["TILE_HEADS"] + 1].copy(),
        "rope": blob.view(np.float32)[b[H["OFF_ROPE"]]: b[H["OFF_ROPE"]] + 128].copy(),
        "off_aux": int(b[H["OFF_AUX"]]),
    }


# ----------------------------------------------------------------------------
# torch helpers (marshalling only)
# ----------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _dtype_code(dt) -> int:
    torch = _torch()
    if dt == torch.float16 or dt == "fp16":
        return ABP_F16
    if dt == torch.bfloat16 or dt == "bf16":
        return ABP_BF16
    if dt == torch.float32 or dt == "fp32":
        return ABP_F32
    raise ValueError(f"unsupported dtype {dt}")


def _torch_dtype(code: int):
    torch = _torch()
    return {ABP_F16: torch.float16, ABP_BF16: torch.bfloat16, ABP_F32: torch.float32}[code]


def make_params(num_qo_heads: int, num_kv_heads: int, head_dim: int, page_size: int, dtype,
                out_dtype=None, sm_scale: float = 0.0, causal: bool = False,
                rope_theta: float = 0.0, rope_llama31=None, kv_fp8: bool = False,
                k_scale: float = 1.0, v_scale: float = 1.0,
                rope_interleave: bool = False) -> AbpParams:
    """abp_params; ``rope_theta`` > 0 turns on the fused LLaMA RoPE, and
    ``rope_llama31 = (factor, low_freq_factor, high_freq_factor, old_context_len)``
    (e.g. ``LLAMA31_ROPE``) its LLaMA 3.1 frequency scaling. ``kv_fp8`` selects
    K/V pages of e4m3 codes worth ``k_scale`` / ``v_scale`` times their values;
    ``rope_interleave`` pairs adjacent elements (2j, 2j + 1) instead of (j, j + d/2)."""
    q = _dtype_code(dtype)
    o = q if out_dtype is None else _dtype_code(out_dtype)
    rope = 0 if rope_theta <= 0 else (2 if rope_llama31 is not None else 1)
    l31 = tuple(float(x) for x in rope_llama31) if rope_llama31 is not None else (0.0,) * 4
    return AbpParams(num_qo_heads, num_kv_heads, head_dim, page_size, q, o, float(sm_scale),
                     int(bool(causal)), rope, float(rope_theta), *l31, int(bool(kv_fp8)),
                     float(k_scale), float(v_scale), int(bool(rope_interleave)))


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _i32_host(a) -> np.ndarray:
    torch = _torch()
    if isinstance(a, torch.Tensor):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=np.int32)


class _Planned:
    """Pinned host + device workspaces and the current plan for one kind."""

    kind = ABP_KIND_DECODE

    def __init__(self, params: AbpParams, max_batch: int, max_qo_tokens: int = 0,
                 num_workers: int = 0, device=None):
        torch = _torch()
        self.params = params
        self.max_batch = int(max_batch)
        self.max_qo_tokens = int(max_qo_tokens)
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None \
            else torch.device(device)
        with torch.cuda.device(self.device):
            # num_workers <= 0: the library picks one worker per resident workgroup slot
            hb, db = abp_workspace_size(self.kind, params, self.max_batch, self.max_qo_tokens,
                                        num_workers)
            self.num_workers = int(num_workers)
            self.host_ws = torch.empty(max(hb, 16), dtype=torch.uint8, pin_memory=True)
            self.dev_ws = torch.empty(max(db, 256), dtype=torch.uint8, device=self.device)
        self.plan_struct = None
        self._upload_done = None

    def _wait_upload(self):
        if self._upload_done is not None:
            self._upload_done.synchronize()

    def _after_upload(self, stream):
        torch = _torch()
        ev = torch.cuda.Event()
        ev.record(stream if stream is not None else torch.cuda.current_stream(self.device))
        self._upload_done = ev


class BatchDecode(_Planned):
    """Batch decode over a paged KV cache: plan on the CPU, run on the GPU."""

    kind = ABP_KIND_DECODE

    def plan(self, kv_indptr, kv_last_page_len, stream=None) -> AbpPlan:
        indptr = _i32_host(kv_indptr)
        lpl = _i32_host(kv_last_page_len)
        self._wait_upload()
        plan = AbpPlan()
        _check(load_library().abp_decode_plan(
            ctypes.byref(self.params), len(indptr) - 1, indptr.ctypes.data, lpl.ctypes.data,
            self.max_batch, self.num_workers, self.host_ws.data_ptr(), self.host_ws.numel(),
            self.dev_ws.data_ptr(), self.dev_ws.numel(), _stream(stream), ctypes.byref(plan)))
        self._after_upload(stream)
        self.plan_struct = plan
        self.batch = len(indptr) - 1
        return plan

    def run(self, q, k_pages, v_pages, kv_indptr, kv_indices, kv_last_page_len, o=None,
            lse=None, q_pos=None, kv_pos_offset=None, stream=None, return_lse: bool = True):
        torch = _torch()
        if self.plan_struct is None:
            raise RuntimeError("plan() must be called before run()")
        if o is None:
            o = torch.empty(q.shape, dtype=_torch_dtype(self.params.out_dtype), device=q.device)
        if lse is None and return_lse:
            lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
        _check(load_library().abp_decode_run(
            ctypes.byref(self.plan_struct), ctypes.byref(self.params), _ptr(q), _ptr(k_pages),
            _ptr(v_pages), _ptr(kv_indptr), _ptr(kv_indices), _ptr(kv_last_page_len),
            _ptr(q_pos), _ptr(kv_pos_offset), _ptr(o), _ptr(lse), self.dev_ws.data_ptr(),
            self.dev_ws.numel(), _stream(stream)))
        return o, lse


class BatchAppend(_Planned):
    """Ragged append / prefill (causal or not) over a paged KV cache."""

    kind = ABP_KIND_APPEND

    def plan(self, qo_indptr, kv_indptr, kv_last_page_len, stream=None) -> AbpPlan:
        qo = _i32_host(qo_indptr)
        indptr = _i32_host(kv_indptr)
        lpl = _i32_host(kv_last_page_len)
        self._wait_upload()
        plan = AbpPlan()
        _check(load_library().abp_append_plan(
            ctypes.byref(self.params), len(indptr) - 1, qo.ctypes.data, indptr.ctypes.data,
            lpl.ctypes.data, self.max_batch, self.max_qo_tokens, self.num_workers,
            self.host_ws.data_ptr(), self.host_ws.numel(), self.dev_ws.data_ptr(),
            self.dev_ws.numel(), _stream(stream), ctypes.byref(plan)))
        self._after_upload(stream)
        self.plan_struct = plan
        return plan

    def run(self, q, k_pages, v_pages, qo_indptr, kv_indptr, kv_indices, kv_last_page_len,
            o=None, lse=None, q_pos=None, kv_pos_offset=None, stream=None,
            return_lse: bool = True):
        torch = _torch()
        if self.plan_struct is None:
            raise RuntimeError("plan() must be called before run()")
        if o is None:
            o = torch.empty(q.shape, dtype=_torch_dtype(self.params.out_dtype), device=q.device)
        if lse is None and return_lse:
            lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
        _check(load_library().abp_append_run(
            ctypes.byref(self.plan_struct), ctypes.byref(self.params), _ptr(q), _ptr(k_pages),
            _ptr(v_pages), _ptr(qo_indptr), _ptr(kv_indptr), _ptr(kv_indices),
            _ptr(kv_last_page_len), _ptr(q_pos), _ptr(kv_pos_offset), _ptr(o), _ptr(lse),
            self.dev_ws.data_ptr(), self.dev_ws.numel(), _stream(stream)))
        return o, lse


class PodAttention:
    """Mixed batches: decode requests and append (prefill) requests of one paged
    KV cache, planned together and run in one launch whose workgroups take the
    decode or the append role (split chosen by the planner, or decode_groups)."""

    def __init__(self, params: AbpParams, max_decode_batch: int, max_append_batch: int,
                 max_qo_tokens: int, num_groups: int = 0, device=None):
        torch = _torch()
        self.params = params
        self.max_decode_batch = int(max_decode_batch)
        self.max_append_batch = int(max_append_batch)
        self.max_qo_tokens = int(max_qo_tokens)
        self.num_groups = int(num_groups)
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None \
            else torch.device(device)
        with torch.cuda.device(self.device):
            hb, db = abp_pod_workspace_size(params, self.max_decode_batch, self.max_append_batch,
                                            self.max_qo_tokens, self.num_groups)
            self.host_ws = torch.empty(max(hb, 16), dtype=torch.uint8, pin_memory=True)
            self.dev_ws = torch.empty(max(db, 256), dtype=torch.uint8, device=self.device)
        self.plan_struct = None
        self._upload_done = None

    def plan(self, d_kv_indptr, d_kv_last_page_len, qo_indptr, a_kv_indptr, a_kv_last_page_len,
             decode_groups: int = 0, stream=None) -> AbpPodPlan:
        torch = _torch()
        arrs, nd, na = _pod_arrays(d_kv_indptr, d_kv_last_page_len, qo_indptr, a_kv_indptr,
                                   a_kv_last_page_len)
        if self._upload_done is not None:
            self._upload_done.synchronize()
        plan = AbpPodPlan()
        _check(load_library().abp_pod_plan(
            ctypes.byref(self.params), nd, arrs[0].ctypes.data, arrs[1].ctypes.data, na,
            arrs[2].ctypes.data, arrs[3].ctypes.data, arrs[4].ctypes.data, self.max_decode_batch,
            self.max_append_batch, self.max_qo_tokens, self.num_groups, int(decode_groups),
            self.host_ws.data_ptr(), self.host_ws.numel(), self.dev_ws.data_ptr(),
            self.dev_ws.numel(), _stream(stream), ctypes.byref(plan)))
        ev = torch.cuda.Event()
        ev.record(stream if stream is not None else torch.cuda.current_stream(self.device))
        self._upload_done = ev
        self.plan_struct = plan
        return plan

    def run(self, q_decode, q_append, k_pages, v_pages, d_kv_indptr, d_kv_indices,
            d_kv_last_page_len, qo_indptr, a_kv_indptr, a_kv_indices, a_kv_last_page_len,
            o_decode=None, lse_decode=None, o_append=None, lse_append=None, stream=None):
        torch = _torch()
        if self.plan_struct is None:
            raise RuntimeError("plan() must be called before run()")
        odt = _torch_dtype(self.params.out_dtype)
        if q_decode is not None and o_decode is None:
            o_decode = torch.empty(q_decode.shape, dtype=odt, device=q_decode.device)
        if q_decode is not None and lse_decode is None:
            lse_decode = torch.empty(q_decode.shape[:2], dtype=torch.float32,
                                     device=q_decode.device)
        if q_append is not None and o_append is None:
            o_append = torch.empty(q_append.shape, dtype=odt, device=q_append.device)
        if q_append is not None and lse_append is None:
            lse_append = torch.empty(q_append.shape[:2], dtype=torch.float32,
                                     device=q_append.device)
        _check(load_library().abp_pod_run(
            ctypes.byref(self.plan_struct), ctypes.byref(self.params), _ptr(q_decode),
            _ptr(q_append), _ptr(k_pages), _ptr(v_pages), _ptr(d_kv_indptr), _ptr(d_kv_indices),
            _ptr(d_kv_last_page_len), _ptr(qo_indptr), _ptr(a_kv_indptr), _ptr(a_kv_indices),
            _ptr(a_kv_last_page_len), _ptr(o_decode), _ptr(lse_decode), _ptr(o_append),
            _ptr(lse_append), self.dev_ws.data_ptr(), self.dev_ws.numel(), _stream(stream)))
        return (o_decode, lse_decode), (o_append, lse_append)


def merge_state(o_a, lse_a, o_b, lse_b, out_dtype=None, o_out=None, lse_out=None, stream=None):
    """Merge two attention states over disjoint key sets (rows = all leading axes)."""
    torch = _torch()
    d = o_a.shape[-1]
    rows = o_a.numel() // d
    od = _dtype_code(o_a.dtype if out_dtype is None else out_dtype)
    if o_out is None:
        o_out = torch.empty(o_a.shape, dtype=_torch_dtype(od), device=o_a.device)
    if lse_out is None:
        lse_out = torch.empty(lse_a.shape, dtype=torch.float32, device=o_a.device)
    _check(load_library().abp_merge_state(_ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b),
                                          _ptr(o_out), _ptr(lse_out), rows, d,
                                          _dtype_code(o_a.dtype), od, _stream(stream)))
    return o_out, lse_out


def merge_states(o, lse, out_dtype=None, stream=None):
    """Merge states stacked on axis 0: o [n, ..., d], lse [n, ...]."""
    torch = _torch()
    n, d = o.shape[0], o.shape[-1]
    rows = o[0].numel() // d if n else 0
    od = _dtype_code(o.dtype if out_dtype is None else out_dtype)
    o_out = torch.empty(o.shape[1:], dtype=_torch_dtype(od), device=o.device)
    lse_out = torch.empty(lse.shape[1:], dtype=torch.float32, device=o.device)
    _check(load_library().abp_merge_states(_ptr(o), _ptr(lse), n, rows, d, _dtype_code(o.dtype),
                                           od, _ptr(o_out), _ptr(lse_out), _stream(stream)))
    return o_out, lse_out


def single_decode_with_kv_cache(q, k, v, sm_scale: float = 0.0, return_lse: bool = False):
    """One query token against a contiguous K/V ``[kv_len, Hkv, d]``.

    The contiguous cache is one BSR page of size kv_len (paged decode with
    batch 1), so this runs the same kernels as ``BatchDecode``.
    """
    torch = _torch()
    kv_len, hkv, d = k.shape
    params = make_params(q.shape[0], hkv, d, max(kv_len, 1), q.dtype, sm_scale=sm_scale)
    dec = BatchDecode(params, max_batch=1, device=q.device)
    n = 1 if kv_len > 0 else 0
    dec.plan(np.array([0, n]), np.array([max(kv_len, 1)]))
    dev = q.device
    idx = torch.zeros(1, dtype=torch.int32, device=dev)
    o, lse = dec.run(q.unsqueeze(0).contiguous(), k.unsqueeze(0).contiguous(),
                     v.unsqueeze(0).contiguous(),
                     torch.tensor([0, n], dtype=torch.int32, device=dev), idx,
                     torch.tensor([max(kv_len, 1)], dtype=torch.int32, device=dev))
    torch.cuda.current_stream(dev).synchronize()   # the planner's workspaces go out of scope
    return (o[0], lse[0]) if return_lse else o[0]


class CascadeDecode:
    """Decode over a shared prefix (one BSR row in large pages) plus per-request
    suffixes (small pages), merged through their attention states.

    The prefix level runs the append kernel with every request's query as one
    row block against the shared prefix (each prefix page is read once for all
    requests); the suffix level runs the decode kernel; one merge launch folds
    both levels' states (direct or split-tile partials). Both levels write fp32
    states.
    """

    def __init__(self, num_qo_heads: int, num_kv_heads: int, head_dim: int, prefix_page_size: int,
                 page_size: int, dtype, max_batch: int, sm_scale: float = 0.0,
                 rope_theta: float = 0.0, num_workers: int = 0, prefix_workers: int = 0,
                 device=None, rope_llama31=None, rope_interleave: bool = False):
        torch = _torch()
        self.dtype = dtype
        self.pre_params = make_params(num_qo_heads, num_kv_heads, head_dim, prefix_page_size,
                                      dtype, out_dtype=torch.float32, sm_scale=sm_scale,
                                      causal=False, rope_theta=rope_theta,
                                      rope_llama31=rope_llama31, rope_interleave=rope_interleave)
        self.suf_params = make_params(num_qo_heads, num_kv_heads, head_dim, page_size, dtype,
                                      out_dtype=torch.float32, sm_scale=sm_scale,
                                      rope_theta=rope_theta, rope_llama31=rope_llama31,
                                      rope_interleave=rope_interleave)
        self.prefix = BatchAppend(self.pre_params, max_batch=1, max_qo_tokens=max_batch,
                                  num_workers=prefix_workers, device=device)
        self.suffix = BatchDecode(self.suf_params, max_batch=max_batch, num_workers=num_workers,
                                  device=device)

    def plan(self, batch: int, prefix_indptr, prefix_last_page_len, kv_indptr, kv_last_page_len,
             stream=None):
        self.batch = batch
        self.prefix.plan(np.array([0, batch]), prefix_indptr, prefix_last_page_len, stream)
        self.suffix.plan(kv_indptr, kv_last_page_len, stream)

    def run(self, q, prefix_k, prefix_v, prefix_qo_indptr, prefix_indptr, prefix_indices,
            prefix_last_page_len, k_pages, v_pages, kv_indptr, kv_indices, kv_last_page_len,
            q_pos=None, kv_pos_offset=None, o=None, lse=None, stream=None, bufs=None):
        """q [B, Hq, d]; prefix_qo_indptr = [0, B] on the device. RoPE: query b at
        q_pos[b], prefix key t at t, suffix key t at kv_pos_offset[b] + t. One
        ``abp_cascade_run``: both levels' kernels, then one merge of their states."""
        torch = _torch()
        if self.prefix.plan_struct is None or self.suffix.plan_struct is None:
            raise RuntimeError("plan() must be called before run()")
        if bufs is None:
            bufs = self.buffers(q)
        o_p, l_p, o_s, l_s = bufs
        if o is None:
            o = torch.empty(q.shape, dtype=self.dtype, device=q.device)
        if lse is None:
            lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
        _check(load_library().abp_cascade_run(
            ctypes.byref(self.prefix.plan_struct), ctypes.byref(self.pre_params),
            self.prefix.dev_ws.data_ptr(), self.prefix.dev_ws.numel(),
            ctypes.byref(self.suffix.plan_struct), ctypes.byref(self.suf_params),
            self.suffix.dev_ws.data_ptr(), self.suffix.dev_ws.numel(), _ptr(q), _ptr(prefix_k),
            _ptr(prefix_v), _ptr(prefix_qo_indptr), _ptr(prefix_indptr), _ptr(prefix_indices),
            _ptr(prefix_last_page_len), _ptr(k_pages), _ptr(v_pages), _ptr(kv_indptr),
            _ptr(kv_indices), _ptr(kv_last_page_len), _ptr(q_pos), _ptr(kv_pos_offset),
            _ptr(o_p), _ptr(l_p), _ptr(o_s), _ptr(l_s), _ptr(o), _ptr(lse),
            _dtype_code(self.dtype), _stream(stream)))
        return o, lse

    @staticmethod
    def buffers(q):
        torch = _torch()
        B, H, d = q.shape
        mk = lambda *s: torch.empty(s, dtype=torch.float32, device=q.device)
        return mk(B, H, d), mk(B, H), mk(B, H, d), mk(B, H)


class BlockSparseAttention:
    """Attention under a block-sparse-row mask over a dense K/V.

    Row block i (queries i*R .. (i+1)*R - 1) sees the column blocks
    ``indices[indptr[i]:indptr[i+1]]`` of C keys each (C = ``params.page_size``).
    The planner turns each row block into an append request whose pages are its
    column blocks, so the run is the MFMA append kernel (``abp_bsr_*``).
    """

    def __init__(self, params: AbpParams, max_row_blocks: int, max_M: int, num_workers: int = 0,
                 device=None):
        torch = _torch()
        self.params = params
        self.max_row_blocks = int(max_row_blocks)
        self.max_M = int(max_M)
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None \
            else torch.device(device)
        with torch.cuda.device(self.device):
            hb, db = abp_workspace_size(ABP_KIND_BSR, params, self.max_row_blocks, self.max_M,
                                        num_workers)
            self.num_workers = int(num_workers)
            self.host_ws = torch.empty(max(hb, 16), dtype=torch.uint8, pin_memory=True)
            self.dev_ws = torch.empty(max(db, 256), dtype=torch.uint8, device=self.device)
        self.plan_struct = None
        self._upload_done = None

    def plan(self, M: int, N: int, R: int, indptr, stream=None) -> AbpPlan:
        torch = _torch()
        ip = _i32_host(indptr)
        if self._upload_done is not None:
            self._upload_done.synchronize()
        plan = AbpPlan()
        _check(load_library().abp_bsr_plan(
            ctypes.byref(self.params), int(M), int(N), int(R), ip.ctypes.data,
            self.max_row_blocks, self.max_M, self.num_workers, self.host_ws.data_ptr(),
            self.host_ws.numel(), self.dev_ws.data_ptr(), self.dev_ws.numel(), _stream(stream),
            ctypes.byref(plan)))
        ev = torch.cuda.Event()
        ev.record(stream if stream is not None else torch.cuda.current_stream(self.device))
        self._upload_done = ev
        self.plan_struct = plan
        return plan

    def run(self, q, k, v, indptr, indices, o=None, lse=None, stream=None,
            return_lse: bool = True):
        """q [M, Hq, d], k / v [N, Hkv, d]; indptr / indices on the device."""
        torch = _torch()
        if self.plan_struct is None:
            raise RuntimeError("plan() must be called before run()")
        if o is None:
            o = torch.empty(q.shape, dtype=_torch_dtype(self.params.out_dtype), device=q.device)
        if lse is None and return_lse:
            lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
        _check(load_library().abp_bsr_run(
            ctypes.byref(self.plan_struct), ctypes.byref(self.params), _ptr(q), _ptr(k), _ptr(v),
            _ptr(indptr), _ptr(indices), _ptr(o), _ptr(lse), self.dev_ws.data_ptr(),
            self.dev_ws.numel(), _stream(stream)))
        return o, lse


def append_paged_kv_cache(k_new, v_new, append_indptr, k_pages, v_pages, kv_indptr, kv_indices,
                          kv_last_page_len, nnz: Optional[int] = None, stream=None) -> None:
    """Write new rows ``k_new / v_new [nnz, Hkv, d]`` (ragged by ``append_indptr``,
    device int32) into the pages, at the last positions of each request of the
    page table (which must already cover them). ``nnz`` defaults to
    ``k_new.shape[0]``."""
    torch = _torch()
    num_pages, page_size, hkv, d = k_pages.shape
    fp8 = k_pages.dtype == torch.float8_e4m3fn
    params = make_params(hkv, hkv, d, page_size, torch.bfloat16 if fp8 else k_pages.dtype,
                         kv_fp8=fp8)
    batch = append_indptr.shape[0] - 1
    n = int(k_new.shape[0] if nnz is None else nnz)
    _check(load_library().abp_append_paged_kv(
        ctypes.byref(params), batch, n, _ptr(k_new), _ptr(v_new), _ptr(append_indptr),
        _ptr(k_pages), _ptr(v_pages), _ptr(kv_indptr), _ptr(kv_indices), _ptr(kv_last_page_len),
        _stream(stream)))
