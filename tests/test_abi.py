"""C-ABI library: loads, exports every declared symbol, validates arguments.

No compute call is made here (there is no GPU in this suite): every call
below fails validation on the host, before anything could be enqueued.
"""
import ctypes
import glob
import os
import re

import pytest

from ring_exact_attention_amd import _bwa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

FAKE = 0x7F0000000000  # an aligned address that is never dereferenced


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(bwa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_bwa.LIB_PATH):
        pytest.skip("libbwa.so not built")
    return _bwa.lib()


def T(B=1, H=2, S=64, D=128, dtype=_bwa.BWA_BF16, ptr=FAKE, strides=None):
    if strides is None:
        strides = (H * S * D, S * D, D)
    return _bwa.Tensor(ptr, dtype, 0, B, H, S, D, *strides)


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(_bwa.EXPORTED) <= set(names)
    assert "bwa_fwd_slot_timers" in names  # the diagnostic header is scanned too
    for name in names:
        assert hasattr(L, name), name
    assert L.bwa_version() == 1


def test_slot_timers_unsupported_in_default_build(L):
    out = (ctypes.c_longlong * 12)()
    n = ctypes.c_int64(-1)
    assert L.bwa_fwd_slot_timers(out, 1, ctypes.byref(n)) == _bwa.BWA_ERR_UNSUPPORTED
    assert n.value == 0
    assert L.bwa_fwd_slot_timers(None, 1, ctypes.byref(n)) == _bwa.BWA_ERR_INVALID_ARG
    assert L.bwa_fwd_slot_timers(out, -1, ctypes.byref(n)) == _bwa.BWA_ERR_INVALID_ARG


def test_status_strings(L):
    assert L.bwa_status_string(0) == b"BWA_OK"
    assert L.bwa_status_string(3) == b"BWA_ERR_WORKSPACE"
    assert L.bwa_status_string(99) == b"BWA_ERR_UNKNOWN"


def ring_fwd(L, q, k, v, o, n=4, sched=0, mode=1, causal=0, scale=0.1, lse=FAKE, ws=None,
             wsb=0):
    args = [None if x is None else ctypes.byref(x) for x in (q, k, v)]
    return L.bwa_ring_fwd(*args, n, sched, mode, causal, scale,
                          None if o is None else ctypes.byref(o), lse, ws, wsb, None)


def expect(L, status, code, fragment):
    assert status == code, (status, L.bwa_last_error())
    assert fragment in L.bwa_last_error().decode()


def test_ring_fwd_validation(L):
    q, k, o = T(S=64), T(S=256), T(S=64)
    E = _bwa
    expect(L, ring_fwd(L, None, k, k, o), E.BWA_ERR_INVALID_ARG, "q is NULL")
    expect(L, ring_fwd(L, T(D=96), T(D=96, S=256), T(D=96, S=256), T(D=96)),
           E.BWA_ERR_UNSUPPORTED, "head dim")
    expect(L, ring_fwd(L, q, k, k, o, n=0), E.BWA_ERR_INVALID_ARG, "shards")
    expect(L, ring_fwd(L, q, k, k, o, n=257), E.BWA_ERR_INVALID_ARG, "shards")
    expect(L, ring_fwd(L, q, k, k, o, causal=1), E.BWA_ERR_UNSUPPORTED, "causal")
    expect(L, ring_fwd(L, q, k, k, o, causal=3), E.BWA_ERR_INVALID_ARG, "causal must be")
    sq = T(S=300)
    expect(L, ring_fwd(L, sq, sq, sq, sq, n=7, causal=2), E.BWA_ERR_UNSUPPORTED, "divide")
    expect(L, ring_fwd(L, q, k, T(S=256, dtype=0), o), E.BWA_ERR_INVALID_ARG, "dtype")
    expect(L, ring_fwd(L, q, k, T(S=255), o), E.BWA_ERR_INVALID_ARG, "lengths differ")
    expect(L, ring_fwd(L, q, k, k, T(S=63)), E.BWA_ERR_INVALID_ARG, "o:")
    expect(L, ring_fwd(L, T(ptr=FAKE + 2), k, k, o), E.BWA_ERR_UNSUPPORTED, "aligned")
    expect(L, ring_fwd(L, T(strides=(64 * 2 * 128, 64 * 128, 100)), k, k, o),
           E.BWA_ERR_UNSUPPORTED, "aligned")
    expect(L, ring_fwd(L, q, k, k, o, scale=0.0), E.BWA_ERR_INVALID_ARG, "scale")
    expect(L, ring_fwd(L, q, k, k, o, scale=float("nan")), E.BWA_ERR_INVALID_ARG, "scale")
    expect(L, ring_fwd(L, q, k, k, o, sched=5), E.BWA_ERR_INVALID_ARG, "schedule")
    expect(L, ring_fwd(L, q, k, k, o, mode=7), E.BWA_ERR_INVALID_ARG, "mode")
    expect(L, ring_fwd(L, q, k, k, o, lse=None), E.BWA_ERR_INVALID_ARG, "lse")
    expect(L, ring_fwd(L, q, T(H=3, S=256), T(H=3, S=256), o), E.BWA_ERR_INVALID_ARG, "head")
    big = T(S=256, strides=(2 * (1 << 23), 1 << 23, 1 << 23))  # 16 MiB rows (bf16)
    expect(L, ring_fwd(L, q, big, k, o), E.BWA_ERR_UNSUPPORTED, "row stride")
    # heads broadcast through zero strides: sizes whose grids would overflow are refused
    z = (0, 0, 0)
    expect(L, ring_fwd(L, T(H=1 << 28, S=64, strides=z), T(H=1 << 28, S=256, strides=z),
                       T(H=1 << 28, S=256, strides=z), T(H=1 << 28, S=64, strides=z)),
           E.BWA_ERR_UNSUPPORTED, "2^33 rows")
    hq, hk = T(H=1 << 21, S=1, strides=z), T(H=1 << 21, S=4096, strides=z)
    expect(L, ring_fwd(L, hq, hk, hk, hq, n=4096), E.BWA_ERR_UNSUPPORTED, "grid above 2^30")


def test_transfer_workspace_covers_both_schedules(L):
    q, k = T(S=2048, H=32), T(S=131072, H=32)
    need = L.bwa_ring_fwd_workspace(ctypes.byref(q), ctypes.byref(k), 8, _bwa.MODE_ROUNDS_TRANSFER)
    o = 32 * 2048 * 128 * 4
    kv = 32 * 131072 * 128 * 2
    assert need >= o + 32 * 2048 * 4 + 2 * (2 * kv)  # stationary (O, L) + two (K, V) slots
    assert need >= 2 * (32 * 2048 * 128 * 2 + o + 32 * 2048 * 4)  # two (Q, O, L) slots


def test_ring_fwd_workspace_checks(L):
    q, k, o = T(S=64), T(S=256), T(S=64)
    need = L.bwa_ring_fwd_workspace(ctypes.byref(q), ctypes.byref(k), 4, _bwa.MODE_ROUNDS)
    assert need == 2 * 64 * 128 * 4
    assert L.bwa_ring_fwd_workspace(ctypes.byref(q), ctypes.byref(k), 4, _bwa.MODE_FUSED) == 0
    split = L.bwa_ring_fwd_workspace(ctypes.byref(q), ctypes.byref(k), 4, _bwa.MODE_SPLIT)
    assert split == 4 * 2 * 64 * 128 * 4 + 4 * 2 * 64 * 4
    assert L.bwa_ring_fwd_workspace(ctypes.byref(q), ctypes.byref(k), 0, _bwa.MODE_SPLIT) == 0
    expect(L, ring_fwd(L, q, k, k, o, mode=_bwa.MODE_ROUNDS, ws=None, wsb=0),
           _bwa.BWA_ERR_WORKSPACE, "workspace")
    expect(L, ring_fwd(L, q, k, k, o, mode=_bwa.MODE_SPLIT, ws=FAKE, wsb=split - 1),
           _bwa.BWA_ERR_WORKSPACE, "workspace")
    expect(L, ring_fwd(L, q, k, k, o, mode=_bwa.MODE_SPLIT, ws=FAKE + 16, wsb=split),
           _bwa.BWA_ERR_WORKSPACE, "256-byte")


def test_empty_query_is_a_noop(L):
    q, o = T(S=0, ptr=0), T(S=0, ptr=0)
    k = T(S=16)
    assert ring_fwd(L, q, k, k, o, lse=None) == _bwa.BWA_OK


def test_partial_fwd_validation(L):
    q, k = T(S=64), T(S=256)
    f = L.bwa_partial_fwd
    E = _bwa
    expect(L, f(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), 0, 65, 0, 16, 0.1, 0, FAKE,
                FAKE, 0, None), E.BWA_ERR_INVALID_ARG, "query range")
    expect(L, f(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), 0, 64, 250, 16, 0.1, 0, FAKE,
                FAKE, 0, None), E.BWA_ERR_INVALID_ARG, "key range")
    expect(L, f(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), 0, 64, 0, 16, 0.1, 0, None,
                FAKE, 0, None), E.BWA_ERR_INVALID_ARG, "NULL")
    expect(L, f(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), 0, 64, 0, 16, 0.1, 0,
                FAKE + 4, FAKE, 0, None), E.BWA_ERR_UNSUPPORTED, "aligned")
    assert f(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), 5, 0, 0, 16, 0.1, 0, None, None,
             0, None) == E.BWA_OK
    # 2^30 heads broadcast through zero strides: the grid would pass 2^30 workgroups
    z = (0, 0, 0)
    hq, hk = T(H=1 << 30, S=1, strides=z), T(H=1 << 30, S=2, strides=z)
    expect(L, f(ctypes.byref(hq), ctypes.byref(hk), ctypes.byref(hk), 0, 1, 0, 2, 0.1, 0, FAKE,
                FAKE, 0, None), E.BWA_ERR_UNSUPPORTED, "grid above 2^30")


def test_merge_validation(L):
    E = _bwa
    o = T(S=8)
    expect(L, L.bwa_merge_partials(0, 0, FAKE, FAKE, ctypes.byref(o), FAKE, None),
           E.BWA_ERR_INVALID_ARG, "n = 0")
    expect(L, L.bwa_merge_partials(2, 3, FAKE, FAKE, ctypes.byref(o), FAKE, None),
           E.BWA_ERR_INVALID_ARG, "schedule")
    expect(L, L.bwa_merge(4, 96, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None), E.BWA_ERR_UNSUPPORTED,
           "D must")
    expect(L, L.bwa_merge(-1, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None),
           E.BWA_ERR_INVALID_ARG, "rows")
    expect(L, L.bwa_merge((1 << 33) + 1, 64, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None),
           E.BWA_ERR_UNSUPPORTED, "2^33 rows")
    expect(L, L.bwa_merge(4, 64, None, FAKE, FAKE, FAKE, FAKE, FAKE, None), E.BWA_ERR_INVALID_ARG,
           "NULL")
    assert L.bwa_merge(0, 64, None, None, None, None, None, None, None) == E.BWA_OK


def test_ring_bwd_validation(L):
    q, k = T(S=64), T(S=256)
    args = lambda **kw: [ctypes.byref(x) for x in (q, k, k, q)] + [FAKE, ctypes.byref(q), 4, 0,
                                                                   kw.get("mode", 1), 0, 0.1] + \
        [ctypes.byref(x) for x in (q, kw.get("dk", k), k)] + [None, 0, None]
    expect(L, L.bwa_ring_bwd(*args(dk=T(S=255))), _bwa.BWA_ERR_INVALID_ARG, "dk")
    expect(L, L.bwa_ring_bwd(*args(mode=_bwa.MODE_ROUNDS_TRANSFER)), _bwa.BWA_ERR_UNSUPPORTED,
           "forward mode")
    qf, kf = T(S=64, dtype=0), T(S=256, dtype=0)
    a = [ctypes.byref(x) for x in (qf, kf, kf, qf)] + [FAKE, ctypes.byref(qf), 4, 0, 1, 0, 0.1] + \
        [ctypes.byref(x) for x in (qf, kf, kf)] + [None, 0, None]
    expect(L, L.bwa_ring_bwd(*a), _bwa.BWA_ERR_UNSUPPORTED, "backward")
    # striped causal order: self-attention with n dividing S
    s = T(S=300)
    a = [ctypes.byref(x) for x in (s, s, s, s)] + [FAKE, ctypes.byref(s), 7, 0, 1, 2, 0.1] + \
        [ctypes.byref(x) for x in (s, s, s)] + [None, 0, None]
    expect(L, L.bwa_ring_bwd(*a), _bwa.BWA_ERR_UNSUPPORTED, "divide")


def test_kv_recompute_validation(L):
    k = T(S=64)
    E = _bwa
    f = L.bwa_kv_recompute
    expect(L, f(FAKE, FAKE, FAKE, 1, 64, 4096, 2, 128, 0, ctypes.byref(k), ctypes.byref(k), None),
           E.BWA_ERR_UNSUPPORTED, "bf16")
    expect(L, f(FAKE, FAKE, FAKE, 1, 64, 100, 2, 128, 1, ctypes.byref(k), ctypes.byref(k), None),
           E.BWA_ERR_UNSUPPORTED, "multiple of 64")
    expect(L, f(FAKE, FAKE, FAKE, 1, 65, 4096, 2, 128, 1, ctypes.byref(k), ctypes.byref(k), None),
           E.BWA_ERR_INVALID_ARG, "shape")
    expect(L, f(None, FAKE, FAKE, 1, 64, 4096, 2, 128, 1, ctypes.byref(k), ctypes.byref(k), None),
           E.BWA_ERR_INVALID_ARG, "NULL")


def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64)
    with pytest.raises(ValueError, match="GPU memory"):
        _bwa.bwa_ring_fwd(q, q, q, n=2)


def test_product_path_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "ring_exact_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "liboracle" not in text and "oracle.c" not in text, f


def test_choose_schedule_matches_oracle(L):
    import oracle
    grid = [(5514, 15279944, 4096, 16, 312e12, 25e9, 2), (65536, 65536, 4096, 16, 1e18, 1e9, 2),
            (1_000_000, 4096, 4096, 8, 312e12, 25e9, 2), (8192, 8192, 4096, 2, 1e9, 1e18, 2),
            (2048, 131072 * 8, 4096, 8, 2.5e15, 153e9, 2), (300, 1000, 128, 4, 1e12, 1e9, 4),
            (1, 1, 1, 1, 1.0, 1.0, 1)]
    for args in grid:
        got, tg = _bwa.bwa_choose_schedule(*args)
        want, tw = oracle.schedule_model(*args)
        assert got == want, args
        for a, b in (("t_compute", "compute"), ("t_comm_kv_stationary", "comm_kv"),
                     ("t_comm_q_stationary", "comm_q"), ("t_round_kv_stationary", "round_kv"),
                     ("t_round_q_stationary", "round_q")):
            assert abs(tg[a] - tw[b]) <= 1e-12 * abs(tw[b]), (args, a)


def test_choose_schedule_validation(L):
    choice = ctypes.c_int32()
    f = L.bwa_choose_schedule
    bad = [(0, 10, 8, 2, 1e12, 1e9, 2), (10, -1, 8, 2, 1e12, 1e9, 2), (10, 10, 8, 0, 1e12, 1e9, 2),
           (10, 10, 8, 2, 0.0, 1e9, 2), (10, 10, 8, 2, 1e12, float("inf"), 2),
           (10, 10, 8, 2, float("nan"), 1e9, 2), (10, 10, 8, 2, 1e12, 1e9, 0)]
    for args in bad:
        assert f(*args, ctypes.byref(choice), None) == _bwa.BWA_ERR_INVALID_ARG, args
    assert f(10, 10, 8, 2, 1e12, 1e9, 2, None, None) == _bwa.BWA_ERR_INVALID_ARG
    assert f(10, 10, 8, 2, 1e12, 1e9, 2, ctypes.byref(choice), None) == _bwa.BWA_OK


def test_kv_recompute_bwd_validation(L):
    f = L.bwa_kv_recompute_bwd
    E = _bwa
    g = T(B=1, H=2, S=128, D=128)
    F = ctypes.c_void_p(FAKE)

    def call(B=1, S=128, Esz=256, H=2, D=128, dk=g, dv=g, outs=(F, F, F)):
        return f(F, F, F, ctypes.byref(dk), ctypes.byref(dv), B, S, Esz, H, D, *outs, 0, None)
    expect(L, call(Esz=192), E.BWA_ERR_UNSUPPORTED, "multiple of 256")
    expect(L, call(S=100, dk=T(S=100), dv=T(S=100)), E.BWA_ERR_UNSUPPORTED, "multiple of 64")
    expect(L, call(H=1, dk=T(H=1, S=128), dv=T(H=1, S=128)), E.BWA_ERR_UNSUPPORTED,
           "H*D must be a multiple of 256")
    expect(L, call(dv=T(S=128, strides=(2 * 128 * 128, 128, 2 * 128))), E.BWA_ERR_UNSUPPORTED,
           "share one layout")
    expect(L, call(outs=(None, None, None)), E.BWA_ERR_INVALID_ARG, "no output")
    expect(L, call(dk=T(S=64)), E.BWA_ERR_INVALID_ARG, "does not match")


def test_binding_rejects_missized_buffers():
    """Buffers the C ABI indexes by row without a size of their own (LSE,
    accumulators, partials, merge outputs) are checked in the binding before
    any pointer reaches the library (host only: the checks raise first)."""
    import torch
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16)
    f = lambda *s: torch.zeros(*s, dtype=torch.float32)
    with pytest.raises(ValueError, match="lse has"):
        _bwa.bwa_ring_fwd(q, k, k, 2, lse=f(1, 2, 7))
    with pytest.raises(ValueError, match="lse must be contiguous float32"):
        _bwa.bwa_ring_fwd(q, k, k, 2, lse=f(1, 2, 16)[:, :, ::2])
    with pytest.raises(ValueError, match="lse has"):
        _bwa.bwa_ring_bwd(q, k, k, q, f(1, 2, 9), q, 2)
    with pytest.raises(ValueError, match="o_acc has"):
        _bwa.bwa_partial_fwd(q, k, k, 0, 8, 0, 16, 0.1, False, f(1, 2, 7, 64), f(1, 2, 8), False)
    with pytest.raises(ValueError, match="lse_acc has"):
        _bwa.bwa_partial_fwd(q, k, k, 0, 8, 0, 16, 0.1, False, f(1, 2, 8, 64), f(1, 2, 9), False)
    with pytest.raises(ValueError, match="holds 3 partials"):
        _bwa.bwa_merge_partials(f(3, 1, 2, 8, 64), f(3, 1, 2, 8), 4)
    with pytest.raises(ValueError, match="lse_parts has"):
        _bwa.bwa_merge_partials(f(3, 1, 2, 8, 64), f(3, 1, 2, 7), 3)
    a, la = f(16, 64), f(16)
    with pytest.raises(ValueError, match="o_out has"):
        _bwa.bwa_merge(a, la, a, la, o_out=f(15, 64), lse_out=f(16))
    with pytest.raises(ValueError, match="o_out must be contiguous float32"):
        _bwa.bwa_merge(a, la, a, la, o_out=a.bfloat16(), lse_out=f(16))
    with pytest.raises(ValueError, match="lse_out has"):
        _bwa.bwa_merge(a, la, a, la, o_out=f(16, 64), lse_out=f(17))


def test_ring_bwd_noalloc_validation(L):
    """Host-side checks of the allocation-free backward, before any device call."""
    def call(S, mode=1, H=2):
        t = T(H=H, S=S)
        return L.bwa_ring_bwd_noalloc(*[ctypes.byref(t)] * 4, FAKE, ctypes.byref(t), 4, 0, mode,
                                      0, 0.1, *[ctypes.byref(t)] * 3, None)
    expect(L, call(64, mode=_bwa.MODE_ROUNDS), _bwa.BWA_ERR_UNSUPPORTED, "ROUNDS")
    expect(L, call(64, mode=_bwa.MODE_ROUNDS_TRANSFER), _bwa.BWA_ERR_UNSUPPORTED, "forward mode")
    # 128 heads x 32769 rows x 4 bytes of Delta exceed the 16 MiB array
    expect(L, call(32769, H=128), _bwa.BWA_ERR_WORKSPACE, "scratch")
    q0, kk = T(S=0), T(S=64)  # empty query: nothing to do, nothing touched
    assert L.bwa_ring_bwd_noalloc(ctypes.byref(q0), ctypes.byref(kk), ctypes.byref(kk),
                                  ctypes.byref(q0), None, ctypes.byref(q0), 4, 0, 1, 0, 0.1,
                                  ctypes.byref(q0), ctypes.byref(kk), ctypes.byref(kk),
                                  None) == _bwa.BWA_OK
