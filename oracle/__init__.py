"""Independent CPU oracle (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package. It shares no code with the HIP library: the
attention oracle is the fp64 definition evaluated by walking the page table,
and ``plan_ref`` is the reference of the work-unit planner.
"""
from .attention import (append_paged_kv, append_workload, attend, attend_masked, bsr_attention,
                        bsr_mask, cascade_decode, decode_workload, fp8_e4m3_to_f64, merge, paged_append,
                        paged_decode, request_kv_len, rope_inv_freq, rope_rotate, storage_to_f64,
                        walk_pages)
from .plan_ref import KIND_APPEND, KIND_DECODE, PlanError, plan_ref

__all__ = [
    "append_paged_kv", "append_workload", "attend", "attend_masked", "bsr_attention", "bsr_mask",
    "cascade_decode", "fp8_e4m3_to_f64", "rope_inv_freq", "decode_workload", "merge", "paged_append",
    "paged_decode", "request_kv_len", "rope_rotate", "storage_to_f64", "walk_pages",
    "KIND_APPEND", "KIND_DECODE", "PlanError", "plan_ref",
]
