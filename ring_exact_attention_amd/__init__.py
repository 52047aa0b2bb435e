"""Blockwise / ring exact attention for AMD MI355X (gfx950).

The compute lives in libbwa.so (HIP kernels behind the C ABI of
include/bwa.h); this package is its thin Python binding.  Importing it does
not load the library; the first call does, and raises if it is not built.
"""
from ._bwa import (  # noqa: F401
    BwaError,
    MODE_FUSED,
    MODE_ROUNDS,
    MODE_SPLIT,
    SCHED_KV_STATIONARY,
    SCHED_Q_STATIONARY,
    bwa_choose_schedule,
    bwa_kv_recompute,
    bwa_kv_recompute_bwd,
    bwa_merge,
    bwa_merge_partials,
    bwa_partial_fwd,
    bwa_ring_bwd,
    bwa_ring_bwd_noalloc,
    bwa_ring_fwd,
    lib,
    ring_bwd_workspace,
    ring_fwd_workspace,
)

__all__ = ["bwa_partial_fwd", "bwa_merge", "bwa_merge_partials", "bwa_ring_fwd", "bwa_ring_bwd",
           "bwa_ring_bwd_noalloc", "bwa_kv_recompute", "bwa_kv_recompute_bwd", "bwa_choose_schedule",
           "BwaError", "lib"]
