"""ctypes binding of libbwa.so (the C ABI in include/bwa.h).

Argument marshalling only: tensors become (pointer, shape, strides) records,
the current torch stream becomes the hipStream_t, and PyTorch allocates the
outputs and workspace.  Every step of the computation runs in the library's
HIP kernels; there is no fallback.  If the library is not built, every call
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbwa.so")
# the same library built with the forward kernel's phase clocks (include/bwa_diag.h)
SLOT_TIMERS_LIB_PATH = os.path.join(_PKG, "libbwa_slot_timers.so")
SLOT_FIELDS = 6

BWA_OK, BWA_ERR_INVALID_ARG, BWA_ERR_UNSUPPORTED, BWA_ERR_WORKSPACE, BWA_ERR_HIP, \
    BWA_ERR_INTERNAL = range(6)
BWA_F32, BWA_BF16 = 0, 1
SCHED_KV_STATIONARY, SCHED_Q_STATIONARY = 0, 1
MODE_ROUNDS, MODE_FUSED, MODE_SPLIT, MODE_ROUNDS_TRANSFER = 0, 1, 2, 3

SCHEDULES = {"kv": SCHED_KV_STATIONARY, "lv": SCHED_KV_STATIONARY, "kv_stationary": 0,
             "q": SCHED_Q_STATIONARY, "ring": SCHED_Q_STATIONARY, "q_stationary": 1}
MODES = {"rounds": MODE_ROUNDS, "fused": MODE_FUSED, "split": MODE_SPLIT,
         "rounds_transfer": MODE_ROUNDS_TRANSFER}

EXPORTED = ("bwa_partial_fwd", "bwa_merge", "bwa_merge_partials", "bwa_ring_fwd_workspace",
            "bwa_ring_fwd",
            "bwa_ring_bwd_workspace", "bwa_ring_bwd", "bwa_ring_bwd_noalloc", "bwa_kv_recompute",
            "bwa_kv_recompute_bwd",
            "bwa_choose_schedule",
            "bwa_status_string",
            "bwa_last_error", "bwa_version", "bwa_fwd_slot_timers")


class ScheduleModel(ctypes.Structure):
    _fields_ = [("t_compute", ctypes.c_double), ("t_comm_kv_stationary", ctypes.c_double),
                ("t_comm_q_stationary", ctypes.c_double),
                ("t_round_kv_stationary", ctypes.c_double),
                ("t_round_q_stationary", ctypes.c_double)]


class BwaError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}")
        self.status = status


class Tensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("B", ctypes.c_int64), ("H", ctypes.c_int64), ("S", ctypes.c_int64),
                ("D", ctypes.c_int64), ("sB", ctypes.c_int64), ("sH", ctypes.c_int64),
                ("sS", ctypes.c_int64)]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m "
                               "ring_exact_attention_amd.build` (or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, f32, ci, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int,
                                ctypes.c_size_t)
        T = ctypes.POINTER(Tensor)
        L.bwa_partial_fwd.argtypes = [T, T, T, i64, i64, i64, i64, f32, ci, vp, vp, ci, vp]
        L.bwa_merge.argtypes = [i64, i64, vp, vp, vp, vp, vp, vp, vp]
        L.bwa_merge_partials.argtypes = [ci, ci, vp, vp, T, vp, vp]
        L.bwa_ring_fwd_workspace.argtypes = [T, T, ci, ci]
        L.bwa_ring_fwd_workspace.restype = sz
        L.bwa_ring_fwd.argtypes = [T, T, T, ci, ci, ci, ci, f32, T, vp, vp, sz, vp]
        L.bwa_ring_bwd_workspace.argtypes = [T, T, ci, ci]
        L.bwa_ring_bwd_workspace.restype = sz
        L.bwa_ring_bwd.argtypes = [T, T, T, T, vp, T, ci, ci, ci, ci, f32, T, T, T, vp, sz, vp]
        L.bwa_ring_bwd_noalloc.argtypes = [T, T, T, T, vp, T, ci, ci, ci, ci, f32, T, T, T, vp]
        L.bwa_kv_recompute.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_int32, T, T,
                                       vp]
        for name in ("bwa_partial_fwd", "bwa_merge", "bwa_merge_partials", "bwa_ring_fwd",
                     "bwa_ring_bwd", "bwa_ring_bwd_noalloc", "bwa_kv_recompute"):
            getattr(L, name).restype = ci
        L.bwa_kv_recompute_bwd.argtypes = [vp, vp, vp, T, T, i64, i64, i64, i64, i64, vp, vp, vp,
                                           ctypes.c_int32, vp]
        L.bwa_choose_schedule.argtypes = [i64, i64, i64, ctypes.c_int32, ctypes.c_double,
                                          ctypes.c_double, ctypes.c_int32,
                                          ctypes.POINTER(ctypes.c_int32),
                                          ctypes.POINTER(ScheduleModel)]
        L.bwa_choose_schedule.restype = ci
        L.bwa_status_string.argtypes = [ci]
        L.bwa_status_string.restype = ctypes.c_char_p
        L.bwa_last_error.restype = ctypes.c_char_p
        L.bwa_version.restype = ci
        L.bwa_fwd_slot_timers.argtypes = [vp, i64, ctypes.POINTER(ctypes.c_int64)]
        L.bwa_fwd_slot_timers.restype = ci
        _lib = L
    return _lib


def use_library(path: str):
    """Load the library from `path` for every later call (for example the
    diagnostic build at SLOT_TIMERS_LIB_PATH); calls already enqueued are not
    affected."""
    global _lib, LIB_PATH
    LIB_PATH = path
    _lib = None
    return lib()


def fwd_slot_timers():
    """Phase clocks of the last bf16 forward launch (diagnostic build only), as
    an int64 array [records, 2 wave groups, SLOT_FIELDS]; see bwa_fwd_slot_timers."""
    import numpy as np
    L = lib()
    n = ctypes.c_int64(0)
    probe = (ctypes.c_longlong * (2 * SLOT_FIELDS))()
    _check(L.bwa_fwd_slot_timers(probe, 0, ctypes.byref(n)))
    out = np.zeros((n.value, 2, SLOT_FIELDS), dtype=np.int64)
    _check(L.bwa_fwd_slot_timers(out.ctypes.data, n.value, ctypes.byref(n)))
    return out


def _check(status: int):
    if status != BWA_OK:
        L = lib()
        raise BwaError(status, L.bwa_status_string(status).decode(),
                       L.bwa_last_error().decode())


def _dtype_code(dt) -> int:
    if dt == torch.bfloat16:
        return BWA_BF16
    if dt == torch.float32:
        return BWA_F32
    raise TypeError(f"dtype {dt} not supported (float32, bfloat16)")


def as_bwa(t: torch.Tensor) -> Tensor:
    """Describe a [B, H, S, D] device tensor (unit stride along D) to the library."""
    _on_device(t)
    if t.dim() != 4:
        raise ValueError("expected a [B, H, S, D] tensor")
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError("the head dimension must have unit stride")
    B, H, S, D = t.shape
    sB, sH, sS, _ = t.stride()
    return Tensor(t.data_ptr() if t.numel() else 0, _dtype_code(t.dtype), 0, B, H, S, D, sB, sH,
                  sS)


def _on_device(t: torch.Tensor):
    if not t.is_cuda:
        raise ValueError("tensors must live in GPU memory (the library takes device pointers)")


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t):
    if t is None:
        return None
    _on_device(t)
    return t.data_ptr()


def _causal(c) -> int:
    """False/True, or "striped" (rows in the striped order over the ring's shards)."""
    if isinstance(c, str):
        if c != "striped":
            raise ValueError(f"unknown causal layout {c!r}")
        return 2
    return int(bool(c))


def _need_f32(name, t, numel):
    """t must be a contiguous float32 device tensor of exactly `numel` elements:
    the library indexes such buffers by row and cannot size-check them."""
    if t.dtype != torch.float32 or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous float32")
    if t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, {numel} expected")


def bwa_partial_fwd(q, k, v, q0, nq, k0, nk, scale, causal, o_acc, lse_acc, accumulate):
    """One block pair merged into (o_acc fp32 [B,H,SQ,D], lse_acc fp32 [B,H,SQ])."""
    B, H, SQ, D = q.shape
    _need_f32("o_acc", o_acc, B * H * SQ * D)
    _need_f32("lse_acc", lse_acc, B * H * SQ)
    tq, tk, tv = as_bwa(q), as_bwa(k), as_bwa(v)
    _check(lib().bwa_partial_fwd(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), q0, nq, k0,
                                 nk, float(scale), _causal(causal), _ptr(o_acc), _ptr(lse_acc),
                                 int(bool(accumulate)), _stream(q.device)))


def bwa_merge(o_a, lse_a, o_b, lse_b, o_out=None, lse_out=None):
    """Rescale-merge two fp32 partials ([..., D], [...]); returns (o_out, lse_out)."""
    for t in (o_a, lse_a, o_b, lse_b):
        if t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("merge inputs must be contiguous float32")
    o_out = torch.empty_like(o_a) if o_out is None else o_out
    lse_out = torch.empty_like(lse_a) if lse_out is None else lse_out
    D = o_a.shape[-1]
    rows = lse_a.numel()
    if o_a.numel() != rows * D or o_b.shape != o_a.shape or lse_b.shape != lse_a.shape:
        raise ValueError("merge operand shapes differ")
    _need_f32("o_out", o_out, rows * D)
    _need_f32("lse_out", lse_out, rows)
    _check(lib().bwa_merge(rows, D, _ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o_out),
                           _ptr(lse_out), _stream(o_a.device)))
    return o_out, lse_out


def bwa_merge_partials(o_parts, lse_parts, n, sched="kv", o=None, lse=None, dtype=None):
    """Merge n per-shard partials (o_parts fp32 [n,B,H,S_Q,D], lse_parts fp32
    [n,B,H,S_Q]) in each query block's ring order; returns (o, lse)."""
    if o_parts.dim() != 5:
        raise ValueError("o_parts must be [n, B, H, S_Q, D]")
    m, B, H, SQ, D = o_parts.shape
    if m != int(n):
        raise ValueError(f"o_parts holds {m} partials, n = {n}")
    _need_f32("o_parts", o_parts, m * B * H * SQ * D)
    _need_f32("lse_parts", lse_parts, m * B * H * SQ)
    if o is None:
        o = torch.empty(B, H, SQ, D, dtype=dtype or torch.float32, device=o_parts.device)
    if lse is None:
        lse = torch.empty(B, H, SQ, dtype=torch.float32, device=o_parts.device)
    if tuple(o.shape) != (B, H, SQ, D):
        raise ValueError("o must be [B, H, S_Q, D] like the partials")
    _need_f32("lse", lse, B * H * SQ)
    to = as_bwa(o)
    _check(lib().bwa_merge_partials(int(n), _sched(sched), _ptr(o_parts), _ptr(lse_parts),
                                    ctypes.byref(to), _ptr(lse), _stream(o_parts.device)))
    return o, lse


def split_workspace_views(workspace, n, B, H, SQ, D):
    """(o_parts, lse_parts) views of a SPLIT-mode forward workspace."""
    a = (n * B * H * SQ * D * 4 + 255) // 256 * 256
    o_parts = workspace[: n * B * H * SQ * D * 4].view(torch.float32).view(n, B, H, SQ, D)
    lse_parts = workspace[a: a + n * B * H * SQ * 4].view(torch.float32).view(n, B, H, SQ)
    return o_parts, lse_parts


def _sched(s) -> int:
    return SCHEDULES[s] if isinstance(s, str) else int(s)


def _mode(m) -> int:
    return MODES[m] if isinstance(m, str) else int(m)


def ring_fwd_workspace(q, k, n, mode) -> int:
    tq, tk = as_bwa(q), as_bwa(k)
    return int(lib().bwa_ring_fwd_workspace(ctypes.byref(tq), ctypes.byref(tk), n, _mode(mode)))


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return None
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace smaller than {nbytes} bytes")
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def bwa_ring_fwd(q, k, v, n, sched="kv", mode="fused", causal=False, scale=None, o=None,
                 lse=None, workspace=None):
    """Ring forward over n shards; returns (o [B,H,SQ,D] q.dtype, lse fp32 [B,H,SQ])."""
    B, H, SQ, D = q.shape
    scale = D ** -0.5 if scale is None else scale
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty(B, H, SQ, dtype=torch.float32, device=q.device) if lse is None else lse
    _need_f32("lse", lse, B * H * SQ)
    m = _mode(mode)
    ws = _workspace(ring_fwd_workspace(q, k, n, m), q.device, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    tq, tk, tv, to = as_bwa(q), as_bwa(k), as_bwa(v), as_bwa(o)
    _check(lib().bwa_ring_fwd(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), int(n),
                              _sched(sched), m, _causal(causal), float(scale), ctypes.byref(to),
                              _ptr(lse), _ptr(ws), nbytes, _stream(q.device)))
    return o, lse


def ring_bwd_workspace(q, k, n, mode) -> int:
    tq, tk = as_bwa(q), as_bwa(k)
    return int(lib().bwa_ring_bwd_workspace(ctypes.byref(tq), ctypes.byref(tk), n, _mode(mode)))


def bwa_ring_bwd(q, k, v, o, lse, dout, n, sched="kv", mode="fused", causal=False, scale=None,
                 dq=None, dk=None, dv=None, workspace=None):
    """Ring backward; returns (dq, dk, dv) in q's dtype."""
    D = q.shape[-1]
    scale = D ** -0.5 if scale is None else scale
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need_f32("lse", lse, q.shape[0] * q.shape[1] * q.shape[2])
    m = _mode(mode)
    ws = _workspace(ring_bwd_workspace(q, k, n, m), q.device, workspace)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    t = [as_bwa(x) for x in (q, k, v, o, dout, dq, dk, dv)]
    _check(lib().bwa_ring_bwd(ctypes.byref(t[0]), ctypes.byref(t[1]), ctypes.byref(t[2]),
                              ctypes.byref(t[3]), _ptr(lse), ctypes.byref(t[4]), int(n),
                              _sched(sched), m, _causal(causal), float(scale),
                              ctypes.byref(t[5]), ctypes.byref(t[6]), ctypes.byref(t[7]),
                              _ptr(ws), nbytes, _stream(q.device)))
    return dq, dk, dv


def bwa_ring_bwd_noalloc(q, k, v, o, lse, dout, n, dq, dk, dv, sched="kv", mode="fused",
                         causal=False, scale=None):
    """bwa_ring_bwd with the library's static scratch array instead of a
    workspace: the caller passes every output; nothing is allocated."""
    D = q.shape[-1]
    scale = D ** -0.5 if scale is None else scale
    _need_f32("lse", lse, q.shape[0] * q.shape[1] * q.shape[2])
    t = [as_bwa(x) for x in (q, k, v, o, dout, dq, dk, dv)]
    _check(lib().bwa_ring_bwd_noalloc(ctypes.byref(t[0]), ctypes.byref(t[1]), ctypes.byref(t[2]),
                                      ctypes.byref(t[3]), _ptr(lse), ctypes.byref(t[4]), int(n),
                                      _sched(sched), _mode(mode), _causal(causal), float(scale),
                                      ctypes.byref(t[5]), ctypes.byref(t[6]), ctypes.byref(t[7]),
                                      _stream(q.device)))
    return dq, dk, dv


def bwa_kv_recompute(y, wk_t, wv_t, H, D, k=None, v=None):
    """K = y W_k, V = y W_v (W given transposed, [H*D, E]); returns (k, v) [B,H,S,D] bf16."""
    B, S, E = y.shape
    for name, t in (("y", y), ("wk_t", wk_t), ("wv_t", wv_t)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k is None:
        k = torch.empty(B, H, S, D, dtype=y.dtype, device=y.device)
    if v is None:
        v = torch.empty(B, H, S, D, dtype=y.dtype, device=y.device)
    tk, tv = as_bwa(k), as_bwa(v)
    _check(lib().bwa_kv_recompute(_ptr(y), _ptr(wk_t), _ptr(wv_t), B, S, E, H, D,
                                  _dtype_code(y.dtype), ctypes.byref(tk), ctypes.byref(tv),
                                  _stream(y.device)))
    return k, v


def bwa_choose_schedule(S_Q, S_KV, d_model, n, flops_per_s, bytes_per_s, elem_bytes=2):
    """Schedule with the shorter modelled round ("kv": LV-XAttn, "q": Ring) and
    the model's times in seconds.  Host-only."""
    L = lib()
    choice = ctypes.c_int32(-1)
    m = ScheduleModel()
    _check(L.bwa_choose_schedule(S_Q, S_KV, d_model, n, float(flops_per_s), float(bytes_per_s),
                                 elem_bytes, ctypes.byref(choice), ctypes.byref(m)))
    times = {f: getattr(m, f) for f, _ in ScheduleModel._fields_}
    return ("kv" if choice.value == SCHED_KV_STATIONARY else "q"), times


def bwa_kv_recompute_bwd(y, wk_t, wv_t, dk, dv, dwk_t=None, dwv_t=None, dy=None,
                         accumulate=False, outputs=("dwk_t", "dwv_t", "dy")):
    """Gradients of K = y W_k, V = y W_v: (dwk_t [H*D, E], dwv_t, dy [B, S, E]), fp32.
    Outputs not passed are allocated (only those named in `outputs`)."""
    for name, t in (("y", y), ("wk_t", wk_t), ("wv_t", wv_t)):
        _on_device(t)
        if not t.is_contiguous() or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a contiguous bf16 tensor")
    B, S, E = y.shape
    H, D = dk.shape[1], dk.shape[3]
    dev = y.device
    if dwk_t is None and "dwk_t" in outputs:
        dwk_t = torch.zeros(H * D, E, dtype=torch.float32, device=dev)
    if dwv_t is None and "dwv_t" in outputs:
        dwv_t = torch.zeros(H * D, E, dtype=torch.float32, device=dev)
    if dy is None and "dy" in outputs:
        dy = torch.zeros(B, S, E, dtype=torch.float32, device=dev)
    for name, t in (("dwk_t", dwk_t), ("dwv_t", dwv_t), ("dy", dy)):
        if t is not None and (not t.is_contiguous() or t.dtype != torch.float32):
            raise ValueError(f"{name} must be a contiguous fp32 tensor")
    L = lib()
    ka, va = as_bwa(dk), as_bwa(dv)
    _check(L.bwa_kv_recompute_bwd(_ptr(y), _ptr(wk_t), _ptr(wv_t), ctypes.byref(ka),
                                  ctypes.byref(va), B, S, E, H, D,
                                  _ptr(dwk_t) if dwk_t is not None else None,
                                  _ptr(dwv_t) if dwv_t is not None else None,
                                  _ptr(dy) if dy is not None else None, 1 if accumulate else 0,
                                  _stream(dev)))
    return dwk_t, dwv_t, dy
