"""fp64 CPU oracle for exact blockwise / ring attention (test infrastructure).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``; never by the product library.
It shares no code with the HIP path.  The arithmetic lives in ``oracle.c``
(plain C, fp64, OpenMP over rows); this module only builds it, marshals
arrays in and out with ctypes, and spells out the round schedule.

Every function follows the definition it cites in ``oracle.c``:

* ``attn_fwd`` -- unblocked softmax(tau Q K^T) V and its row log-sum-exp, the
  result the LV-XAttn review ("Assumptions": online-softmax rescaling is exact)
  and the Ring Attention abstract ("without resorting to approximations") say
  the blockwise methods reach exactly.
* ``attn_partial`` / ``merge`` / ``ring_fwd`` -- the per-pair partials, the
  FlashAttention-style rescale-merge and the n-round ring loop of the LV-XAttn
  review ("What carries the argument"; Figure 3 / Algorithm 1 caption).
* ``attn_bwd`` -- the exact gradient the review's referee report (major
  comment 1) asks the distributed backward to match.
* ``kv_proj`` -- K = y W_k, V = y W_v from the one shared copy of the visual
  features ("What carries the argument", activation recomputation).

Pins: ``tests/test_oracle.py`` checks every function against brute force,
closed forms, invariants and independent library routines.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F64, F32, BF16 = 0, 1, 2
SCHED_KV_STATIONARY, SCHED_Q_STATIONARY = 0, 1

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (IEEE semantics, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-Wall",
             "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        lib = ctypes.CDLL(_LIB)
        i64, f64, vp, ci = ctypes.c_int64, ctypes.c_double, ctypes.c_void_p, ctypes.c_int
        lib.orc_num_threads.restype = ci
        lib.orc_attn_fwd_rows.argtypes = [vp, vp, vp, ci, i64, i64, i64, i64, i64, f64, ci,
                                          vp, i64, vp, vp]
        lib.orc_attn_partial.argtypes = [vp, vp, vp, ci, i64, i64, i64, i64, i64, f64, ci,
                                         i64, i64, i64, i64, vp, vp]
        lib.orc_merge.argtypes = [i64, i64, vp, vp, vp, vp, vp, vp]
        lib.orc_shard_start.argtypes = [i64, i64, i64]
        lib.orc_shard_start.restype = i64
        lib.orc_ring_pair.argtypes = [ci, i64, i64, i64, ctypes.POINTER(i64), ctypes.POINTER(i64)]
        lib.orc_ring_fwd.argtypes = [vp, vp, vp, ci, i64, i64, i64, i64, i64, f64, ci, i64, ci,
                                     vp, vp]
        lib.orc_attn_bwd_heads.argtypes = [vp, vp, vp, vp, ci, ci, i64, i64, i64, i64, i64, f64,
                                           ci, vp, i64, vp, i64, vp, vp, vp, vp, vp]
        lib.orc_kv_proj_rows.argtypes = [vp, vp, ci, i64, i64, i64, i64, vp, i64, vp]
        lib.orc_kv_grad_w_rows.argtypes = [vp, vp, ci, i64, i64, i64, i64, i64, vp, i64, vp]
        lib.orc_kv_grad_y_rows.argtypes = [vp, vp, vp, vp, ci, i64, i64, i64, i64, i64, vp, i64,
                                           vp]
        lib.orc_schedule_model.argtypes = [f64] * 7 + [vp]
        lib.orc_schedule_model.restype = ci
        _lib = lib
    return _lib


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use."""
    return int(_load().orc_num_threads())


def _arr(x):
    """(pointer, dtype code, keep-alive) for a contiguous f64/f32 array or a bf16 tensor.

    bf16 tensors are passed as their raw 16-bit patterns; the C side widens
    them exactly.  Only reinterpretation happens here, no arithmetic.
    """
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().contiguous()
            if x.dtype == torch.bfloat16:
                a = x.view(torch.int16).numpy()
                return a.ctypes.data, BF16, a
            x = x.numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(x)
    if a.dtype == np.float64:
        return a.ctypes.data, F64, a
    if a.dtype == np.float32:
        return a.ctypes.data, F32, a
    raise TypeError(f"oracle input dtype {a.dtype} not supported")


def _same_dtype(*codes):
    if len(set(codes)) != 1:
        raise TypeError("q, k, v must share one dtype")
    return codes[0]


def _causal_code(causal) -> int:
    """0: none; 1: positions in row order; ("striped", n): rows in the striped
    order over n shards (shard w holds positions w, w+n, ...), encoded -n."""
    if isinstance(causal, tuple):
        kind, n = causal
        if kind != "striped" or int(n) < 1:
            raise ValueError("causal must be a bool or ('striped', n)")
        return -int(n)
    return int(bool(causal))


def attn_fwd(q, k, v, scale: float, causal=False, rows=None):
    """Unblocked attention.  q [B,H,SQ,D], k/v [B,H,SKV,D].

    rows=None returns (O [B,H,SQ,D], LSE [B,H,SQ]) in float64; otherwise rows is
    a sequence of flat row indices (b*H + h)*SQ + i and the result is
    (O [len(rows), D], LSE [len(rows)]).
    """
    B, H, SQ, D = q.shape
    SKV = k.shape[2]
    pq, dq, kq = _arr(q)
    pk, dk, kk = _arr(k)
    pv, dv, kv = _arr(v)
    dt = _same_dtype(dq, dk, dv)
    if rows is None:
        nrows, prow, keep = B * H * SQ, None, None
    else:
        keep = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows, prow = keep.size, keep.ctypes.data
    o = np.zeros((nrows, D), np.float64)
    lse = np.zeros((nrows,), np.float64)
    _load().orc_attn_fwd_rows(pq, pk, pv, dt, B, H, SQ, SKV, D, float(scale),
                              _causal_code(causal), prow, nrows, o.ctypes.data, lse.ctypes.data)
    del kq, kk, kv, keep
    if rows is None:
        return o.reshape(B, H, SQ, D), lse.reshape(B, H, SQ)
    return o, lse


def attn_partial(q, k, v, scale: float, causal: bool, q0: int, q1: int, k0: int, k1: int):
    """Partial (O_p, L_p) of query rows [q0,q1) over keys [k0,k1).

    Returns full-size float64 arrays [B,H,SQ,D] / [B,H,SQ]; rows outside
    [q0,q1) hold (0, -inf), the merge identity.
    """
    B, H, SQ, D = q.shape
    SKV = k.shape[2]
    pq, dq, kq = _arr(q)
    pk, dk, kk = _arr(k)
    pv, dv, kv = _arr(v)
    dt = _same_dtype(dq, dk, dv)
    o = np.zeros((B, H, SQ, D), np.float64)
    lse = np.full((B, H, SQ), -np.inf, np.float64)
    _load().orc_attn_partial(pq, pk, pv, dt, B, H, SQ, SKV, D, float(scale), int(causal),
                             q0, q1, k0, k1, o.ctypes.data, lse.ctypes.data)
    del kq, kk, kv
    return o, lse


def merge(oa, la, ob, lb):
    """Rescale-merge of two partials (float64 arrays; O [..., D], L [...])."""
    oa = np.ascontiguousarray(oa, dtype=np.float64)
    ob = np.ascontiguousarray(ob, dtype=np.float64)
    la = np.ascontiguousarray(la, dtype=np.float64)
    lb = np.ascontiguousarray(lb, dtype=np.float64)
    D = oa.shape[-1]
    rows = la.size
    o = np.empty_like(oa)
    lo = np.empty_like(la)
    _load().orc_merge(rows, D, oa.ctypes.data, la.ctypes.data, ob.ctypes.data, lb.ctypes.data,
                      o.ctypes.data, lo.ctypes.data)
    return o, lo


def shard_start(S: int, n: int, k: int) -> int:
    return int(_load().orc_shard_start(S, n, k))


def shard_bounds(S: int, n: int):
    """[(start, end)] of the n shards of a length-S sequence."""
    return [(shard_start(S, n, k), shard_start(S, n, k + 1)) for k in range(n)]


def ring_pair(sched: int, n: int, r: int, w: int):
    """(query block, KV shard) that virtual worker w holds in round r."""
    qb, kb = ctypes.c_int64(), ctypes.c_int64()
    _load().orc_ring_pair(int(sched), n, r, w, ctypes.byref(qb), ctypes.byref(kb))
    return int(qb.value), int(kb.value)


def ring_fwd(q, k, v, scale: float, n: int, sched: int, causal: bool = False):
    """The n-round ring forward with rescale-merge; returns float64 (O, LSE)."""
    B, H, SQ, D = q.shape
    SKV = k.shape[2]
    pq, dq, kq = _arr(q)
    pk, dk, kk = _arr(k)
    pv, dv, kv = _arr(v)
    dt = _same_dtype(dq, dk, dv)
    o = np.zeros((B, H, SQ, D), np.float64)
    lse = np.zeros((B, H, SQ), np.float64)
    _load().orc_ring_fwd(pq, pk, pv, dt, B, H, SQ, SKV, D, float(scale), int(causal), n,
                         int(sched), o.ctypes.data, lse.ctypes.data)
    del kq, kk, kv
    return o, lse


def attn_bwd(q, k, v, do, scale: float, causal=False, heads=None, keys=None):
    """Exact gradient of softmax(tau Q K^T) V for the listed heads (flat b*H+h).
    causal as in attn_fwd (False, True or ("striped", n)).

    Returns dict of float64 arrays: dq [nh,SQ,D], dk/dv [nh,nkeys,D],
    lse/delta [nh,SQ].  heads=None means every head; keys=None every key.
    """
    B, H, SQ, D = q.shape
    SKV = k.shape[2]
    pq, dq_, kq = _arr(q)
    pk, dk_, kk = _arr(k)
    pv, dv_, kv = _arr(v)
    pd, ddo, kd = _arr(do)
    dt = _same_dtype(dq_, dk_, dv_)
    hs = np.arange(B * H, dtype=np.int64) if heads is None else np.asarray(heads, np.int64)
    hs = np.ascontiguousarray(hs)
    nh = hs.size
    if keys is None:
        ks, pks, nk = None, None, SKV
    else:
        ks = np.ascontiguousarray(np.asarray(keys, np.int64))
        pks, nk = ks.ctypes.data, ks.size
    out = dict(dq=np.zeros((nh, SQ, D)), dk=np.zeros((nh, nk, D)), dv=np.zeros((nh, nk, D)),
               lse=np.zeros((nh, SQ)), delta=np.zeros((nh, SQ)))
    _load().orc_attn_bwd_heads(pq, pk, pv, pd, dt, ddo, B, H, SQ, SKV, D, float(scale),
                               _causal_code(causal), hs.ctypes.data, nh, pks,
                               nk if keys is not None else 0,
                               out["dq"].ctypes.data, out["dk"].ctypes.data,
                               out["dv"].ctypes.data, out["lse"].ctypes.data,
                               out["delta"].ctypes.data)
    del kq, kk, kv, kd
    return out


def kv_proj(y, w_t, H: int, D: int, rows=None):
    """K = y W for W = w_t^T (w_t is [H*D, E]); y [B,S,E].

    rows=None returns [B,H,S,D] (head split: head h is columns h*D..h*D+D-1 of
    y W); otherwise rows are flat (b*S + s) indices and the result is
    [len(rows), H*D] in (h, d) order.
    """
    B, S, E = y.shape
    HD = w_t.shape[0]
    if HD != H * D or w_t.shape[1] != E:
        raise ValueError("w_t must be [H*D, E]")
    py, dy, ky = _arr(y)
    pw, dw, kw = _arr(w_t)
    dt = _same_dtype(dy, dw)
    if rows is None:
        nrows, prow, keep = B * S, None, None
    else:
        keep = np.ascontiguousarray(np.asarray(rows, np.int64))
        nrows, prow = keep.size, keep.ctypes.data
    out = np.zeros((nrows, HD), np.float64)
    _load().orc_kv_proj_rows(py, pw, dt, B, S, E, HD, prow, nrows, out.ctypes.data)
    del ky, kw, keep
    if rows is None:
        return out.reshape(B, S, H, D).transpose(0, 2, 1, 3).copy()
    return out


def schedule_model(S_Q, S_KV, d, n, flops_per_s, bytes_per_s, elem_bytes=2):
    """Per-round cost model of the two schedules (LV-XAttn review, "What
    carries the argument").  Returns ("kv" | "q", {compute, comm_kv, comm_q,
    round_kv, round_q} in seconds); "kv" (LV-XAttn) wins ties."""
    out = np.zeros(5, dtype=np.float64)
    c = _load().orc_schedule_model(float(S_Q), float(S_KV), float(d), float(n),
                                   float(flops_per_s), float(bytes_per_s), float(elem_bytes),
                                   out.ctypes.data)
    keys = ("compute", "comm_kv", "comm_q", "round_kv", "round_q")
    return ("kv" if c == 0 else "q"), dict(zip(keys, out.tolist()))


def _rows_arg(rows):
    if rows is None:
        return None, -1, None
    keep = np.ascontiguousarray(np.asarray(rows, np.int64))
    return keep.ctypes.data, keep.size, keep


def kv_grad_w(y, g, rows=None):
    """dW_t[n, e] = sum_{b,s} g[b,h,s,d] y[b,s,e] (n = h*D + d): the gradient of
    w_t ([H*D, E]) for K = y W, W = w_t^T, given dK = g [B,H,S,D].  rows selects
    rows n; returns [len(rows) or H*D, E]."""
    B, S, E = y.shape
    _, H, S2, D = g.shape
    if S2 != S or g.shape[0] != B:
        raise ValueError("g must be [B, H, S, D] matching y [B, S, E]")
    py, dy_, ky = _arr(y)
    pg, dg, kg = _arr(g)
    if dy_ != dg:
        raise ValueError("y and g must share a dtype")
    pr, nr, keep = _rows_arg(rows)
    out = np.zeros((H * D if nr < 0 else nr, E), np.float64)
    _load().orc_kv_grad_w_rows(py, pg, dg, B, S, E, H, D, pr, nr, out.ctypes.data)
    del ky, kg, keep
    return out


def kv_grad_y(gk, gv, wk_t, wv_t, rows=None):
    """dy[b, s, e] = sum_n gk[b,h,s,d] wk_t[n,e] + gv[b,h,s,d] wv_t[n,e]: the
    gradient of y through both projections.  rows selects flat rows b*S + s;
    returns [len(rows) or B*S, E]."""
    B, H, S, D = gk.shape
    E = wk_t.shape[1]
    ptrs = [_arr(t) for t in (gk, gv, wk_t, wv_t)]
    if len({p[1] for p in ptrs}) != 1:
        raise ValueError("inputs must share a dtype")
    pr, nr, keep = _rows_arg(rows)
    out = np.zeros((B * S if nr < 0 else nr, E), np.float64)
    _load().orc_kv_grad_y_rows(ptrs[0][0], ptrs[1][0], ptrs[2][0], ptrs[3][0], ptrs[0][1], B, S, E,
                               H, D, pr, nr, out.ctypes.data)
    del ptrs, keep
    return out
