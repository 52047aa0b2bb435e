"""GPU forward parity: HIP path (through the C ABI) vs the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

from tests.parity import check_fwd, sample_rows, to64

pytestmark = pytest.mark.gpu

MODES = ["rounds", "fused", "split", "rounds_transfer"]
SCHEDS = ["kv", "q"]


@pytest.fixture(scope="module")
def bwa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_exact_attention_amd as m
    m.lib()  # raises if the HIP library is not built
    return m


def gen(B, H, SQ, SKV, D, dtype, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(B, H, SQ, D, generator=g) * std).to(dtype)
    k = (torch.randn(B, H, SKV, D, generator=g) * std).to(dtype)
    v = torch.randn(B, H, SKV, D, generator=g).to(dtype)
    return q, k, v


def log_case(**kw):
    print("case:", " ".join(f"{a}={b}" for a, b in kw.items()), flush=True)


# ------------------------------------------------------------------ tiny fp32 workload

def test_tiny_f32_all_modes(bwa, orc):
    from ring_exact_attention_amd.inputs import WORKLOADS, make_qkv
    w = WORKLOADS["tiny_f32"]
    q, k, v = make_qkv(w)
    O, L = orc.attn_fwd(q, k, v, w.scale)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    for mode in MODES:
        for sched in SCHEDS:
            log_case(test="tiny_f32", mode=mode, sched=sched)
            o, lse = bwa.bwa_ring_fwd(qd, kd, vd, w.n, sched, mode, scale=w.scale)
            torch.cuda.synchronize()
            check_fwd(o, lse, O, L, "f32", f"tiny_f32 {mode}/{sched}")


def test_tiny_f32_partials_and_merge(bwa, orc):
    """The tiny workload as the pages describe one worker's view: four block
    partials from bwa_partial_fwd merged with bwa_merge, and the same chain
    with in-kernel accumulation."""
    from ring_exact_attention_amd.inputs import WORKLOADS, make_qkv
    w = WORKLOADS["tiny_f32"]
    q, k, v = make_qkv(w)
    O, L = orc.attn_fwd(q, k, v, w.scale)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    B, H, SQ, D = q.shape
    bounds = orc.shard_bounds(w.SKV, w.n)
    parts = []
    for a, b in bounds:
        o = torch.zeros(B, H, SQ, D, device="cuda")
        l = torch.zeros(B, H, SQ, device="cuda")
        bwa.bwa_partial_fwd(qd, kd, vd, 0, SQ, a, b - a, w.scale, False, o, l, accumulate=False)
        parts.append((o, l))
        Op, Lp = orc.attn_partial(q, k, v, w.scale, False, 0, SQ, a, b)
        torch.cuda.synchronize()
        check_fwd(o, l, Op, Lp, "f32", f"partial [{a},{b})")
    acc_o, acc_l = parts[0][0].clone(), parts[0][1].clone()
    for o, l in parts[1:]:
        bwa.bwa_merge(acc_o, acc_l, o, l, acc_o, acc_l)  # in place: outputs alias input a
    torch.cuda.synchronize()
    check_fwd(acc_o, acc_l, O, L, "f32", "merge chain")
    o = torch.zeros(B, H, SQ, D, device="cuda")
    l = torch.zeros(B, H, SQ, device="cuda")
    for i, (a, b) in enumerate(reversed(bounds)):
        bwa.bwa_partial_fwd(qd, kd, vd, 0, SQ, a, b - a, w.scale, False, o, l, accumulate=i > 0)
    torch.cuda.synchronize()
    check_fwd(o, l, O, L, "f32", "accumulate chain")


# ------------------------------------------------------------------ small bf16 shapes

SHAPES = [
    # B, H, SQ, SKV, D, n
    (1, 2, 300, 1000, 128, 4),   # ragged tiles and shards
    (2, 1, 64, 64, 64, 1),       # one shard, D = 64
    (1, 1, 1, 7, 128, 7),        # one query, one key per shard
    (1, 3, 517, 1500, 128, 8),
    (1, 2, 20, 2048, 128, 16),   # query blocks of one or two rows
    (1, 1, 5, 100, 128, 8),      # more shards than query rows: empty query blocks
    (2, 2, 256, 4096, 128, 8),   # full tiles
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bf16_shapes_all_modes(bwa, orc, shape):
    B, H, SQ, SKV, D, n = shape
    q, k, v = gen(B, H, SQ, SKV, D, torch.bfloat16, seed=sum(shape))
    scale = 1 / math.sqrt(D)
    O, L = orc.attn_fwd(q, k, v, scale)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    for mode in MODES:
        for sched in SCHEDS:
            log_case(shape=shape, mode=mode, sched=sched)
            o, lse = bwa.bwa_ring_fwd(qd, kd, vd, n, sched, mode, scale=scale)
            torch.cuda.synchronize()
            check_fwd(o, lse, O, L, "bf16", f"{shape} {mode}/{sched}")


@pytest.mark.parametrize("shape", [(1, 2, 700, 128, 4), (1, 1, 300, 64, 3), (1, 2, 1024, 128, 8),
                                   (1, 1, 65, 128, 65)],
                         ids=lambda s: "x".join(map(str, s)))
def test_bf16_causal_all_modes(bwa, orc, shape):
    B, H, S, D, n = shape
    q, k, v = gen(B, H, S, S, D, torch.bfloat16, seed=7 + S)
    scale = 1 / math.sqrt(D)
    O, L = orc.attn_fwd(q, k, v, scale, causal=True)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    for mode in MODES:
        for sched in SCHEDS:
            log_case(causal_shape=shape, mode=mode, sched=sched)
            o, lse = bwa.bwa_ring_fwd(qd, kd, vd, n, sched, mode, causal=True, scale=scale)
            torch.cuda.synchronize()
            check_fwd(o, lse, O, L, "bf16", f"causal {shape} {mode}/{sched}")


def test_f32_causal_and_d128(bwa, orc):
    for (S, D, n, causal) in [(200, 128, 3, True), (96, 64, 5, True), (77, 128, 2, False)]:
        q, k, v = gen(1, 2, S, S + (0 if causal else 33), D, torch.float32, seed=S)
        O, L = orc.attn_fwd(q, k, v, 0.1, causal=causal)
        for mode in MODES:
            log_case(f32=(S, D, n, causal), mode=mode)
            o, lse = bwa.bwa_ring_fwd(q.cuda(), k.cuda(), v.cuda(), n, "q", mode, causal=causal,
                                      scale=0.1)
            torch.cuda.synchronize()
            check_fwd(o, lse, O, L, "f32", f"f32 {S} {D} {mode}")


def test_partial_fully_masked_rows(bwa, orc):
    """Causal pair whose keys all lie after some of its rows: those rows get (0, -inf)."""
    q, k, v = gen(1, 2, 256, 256, 128, torch.bfloat16, seed=3)
    o = torch.full((1, 2, 256, 128), 7.0, device="cuda")
    l = torch.full((1, 2, 256), 7.0, device="cuda")
    bwa.bwa_partial_fwd(q.cuda(), k.cuda(), v.cuda(), 0, 256, 100, 80, 0.125, True, o, l, False)
    torch.cuda.synchronize()
    Op, Lp = orc.attn_partial(q, k, v, 0.125, True, 0, 256, 100, 180)
    check_fwd(o, l, Op, Lp, "bf16", "partial causal")
    assert torch.all(l[:, :, :100] == -math.inf)
    assert torch.all(o[:, :, :100] == 0)


def test_strided_layouts_and_guard_bands(bwa, orc):
    """[B, S, H, D] storage viewed as [B, H, S, D]; output written into the
    middle of a NaN-filled buffer must leave the rest untouched."""
    B, H, SQ, SKV, D, n = 2, 3, 130, 700, 128, 4
    q, k, v = gen(B, H, SQ, SKV, D, torch.bfloat16, seed=11)
    O, L = orc.attn_fwd(q, k, v, 0.09)
    qs = q.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    ks = k.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    vs = v.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    big = torch.full((B, SQ + 8, H, D + 64), float("nan"), dtype=torch.bfloat16, device="cuda")
    o = big[:, 4:4 + SQ, :, 32:32 + D].transpose(1, 2)
    for mode in MODES:
        big.fill_(float("nan"))
        log_case(strided=mode)
        _, lse = bwa.bwa_ring_fwd(qs, ks, vs, n, "kv", mode, scale=0.09, o=o)
        torch.cuda.synchronize()
        check_fwd(o, lse, O, L, "bf16", f"strided {mode}")
        mask = torch.ones_like(big, dtype=torch.bool)
        mask[:, 4:4 + SQ, :, 32:32 + D] = False
        assert torch.isnan(big[mask].float()).all(), "write outside the output view"


def test_hot_rows_peaked_softmax(bwa, orc):
    """1% of K rows scaled by 8 (peaked softmax): the absolute bound bites here."""
    from ring_exact_attention_amd.inputs import WORKLOADS, make_qkv
    w = WORKLOADS["shortq_256_256k"].resized(B=1, H=2, SKV=8192, n=8)
    q, k, v = make_qkv(w)
    O, L = orc.attn_fwd(q, k, v, w.scale)
    for mode in MODES:
        log_case(hot=mode)
        o, lse = bwa.bwa_ring_fwd(q.cuda(), k.cuda(), v.cuda(), w.n, "kv", mode, scale=w.scale)
        torch.cuda.synchronize()
        check_fwd(o, lse, O, L, "bf16", f"hot rows {mode}")


@pytest.mark.parametrize("profile", ["ramp", "jumps"])
def test_scores_growing_across_tiles(bwa, orc, profile):
    """Key norms that grow along the sequence (ramp: x1 to x7; jumps: every
    fifth 64-key tile x6), so that a row's maximum keeps rising from tile to
    tile: the kernel must move its reference and rescale many times, and
    between moves accept probabilities far above 1 relative to it."""
    B, H, SQ, SKV, D = 1, 2, 96, 4096, 128
    g = torch.Generator().manual_seed(17)
    q = torch.randn(B, H, SQ, D, generator=g)
    k = torch.randn(B, H, SKV, D, generator=g)
    j = torch.arange(SKV, dtype=torch.float32)
    f = 1 + 6 * j / SKV if profile == "ramp" else torch.where((j // 64) % 5 == 4, 6.0, 1.0)
    k = k * f[None, None, :, None]
    v = torch.randn(B, H, SKV, D, generator=g)
    q, k, v = q.bfloat16(), k.bfloat16(), v.bfloat16()
    scale = 1 / math.sqrt(D)
    O, L = orc.attn_fwd(q, k, v, scale)
    for n in (1, 4):
        for mode in MODES:
            log_case(profile=profile, n=n, mode=mode)
            o, lse = bwa.bwa_ring_fwd(q.cuda(), k.cuda(), v.cuda(), n, "kv", mode, scale=scale)
            torch.cuda.synchronize()
            check_fwd(o, lse, O, L, "bf16", f"{profile} n={n} {mode}")


def test_deterministic(bwa):
    q, k, v = (x.cuda() for x in gen(1, 4, 512, 4096, 128, torch.bfloat16, seed=5))
    for mode in MODES:
        a = bwa.bwa_ring_fwd(q, k, v, 8, "kv", mode)
        b = bwa.bwa_ring_fwd(q, k, v, 8, "kv", mode)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), mode


def test_slot_timer_build_is_bitwise_default(bwa):
    """The diagnostic build (phase clocks in the forward kernel) computes what
    the default build computes, bit for bit, and records every workgroup's
    tiles: in split mode at n = 4 over 512 rows x 4096 keys a workgroup takes
    256 query rows against one KV shard, so 2 heads x 4 shards x 2 row tiles
    = 16 workgroups, each walking 1024 / 64 = 16 key tiles."""
    from ring_exact_attention_amd import _bwa
    q, k, v = (x.cuda() for x in gen(1, 2, 512, 4096, 128, torch.bfloat16, seed=41))
    qc, kc, vc = (x.cuda() for x in gen(1, 2, 1024, 1024, 128, torch.bfloat16, seed=42))
    default = _bwa.LIB_PATH
    ref = [bwa.bwa_ring_fwd(q, k, v, 4, "kv", "split"),
           bwa.bwa_ring_fwd(qc, kc, vc, 4, "q", "fused", causal=True)]
    torch.cuda.synchronize()
    try:
        _bwa.use_library(_bwa.SLOT_TIMERS_LIB_PATH)
        log_case(test="slot_timers", mode="split")
        o, lse = bwa.bwa_ring_fwd(q, k, v, 4, "kv", "split")
        rec = _bwa.fwd_slot_timers()
        assert torch.equal(o, ref[0][0]) and torch.equal(lse, ref[0][1])
        live = rec[rec[:, 0, 5] > 0]
        assert len(live) == 16
        assert (live[:, :, 5] == 16).all()
        assert (live[:, :, :5] >= 0).all() and (live[:, :, 3] > 0).all()
        log_case(test="slot_timers", mode="fused", causal=True)
        o, lse = bwa.bwa_ring_fwd(qc, kc, vc, 4, "q", "fused", causal=True)
        rec = _bwa.fwd_slot_timers()
        assert torch.equal(o, ref[1][0]) and torch.equal(lse, ref[1][1])
        assert rec[:, :, 5].sum() > 0
    finally:
        _bwa.use_library(default)


def test_schedules_agree_closely(bwa, orc):
    """Both schedules and all modes compute the same pairs.  They differ in
    fp32 merge order and, more, in the reference maximum each probability is
    taken against before it is rounded to bf16 (a shard's own maximum in
    split mode, the running maximum, moved lazily, in fused and rounds mode),
    so each P_ij carries an independent rounding: every element agrees with
    the fused KV-stationary result within 6 sigma of that difference plus one
    bf16 ulp (tests/parity.py, check_modes_agree)."""
    from tests.parity import check_modes_agree, mode_sigma
    qc, kc, vc = gen(1, 2, 512, 8192, 128, torch.bfloat16, seed=9)
    scale = 1 / math.sqrt(128)
    _, L = orc.attn_fwd(qc, kc, vc, scale)
    f64 = lambda t: t.double().numpy().reshape(-1, t.shape[2], t.shape[3])
    sigma = mode_sigma(f64(qc), f64(kc), f64(vc), scale, L.reshape(-1, 512)).reshape(1, 2, 512, 128)
    q, k, v = qc.cuda(), kc.cuda(), vc.cuda()
    ref = bwa.bwa_ring_fwd(q, k, v, 8, "kv", "fused", scale=scale)[0]
    for mode in MODES:
        for sched in SCHEDS:
            o = bwa.bwa_ring_fwd(q, k, v, 8, sched, mode, scale=scale)[0]
            torch.cuda.synchronize()
            check_modes_agree(o, ref, sigma, f"{mode}/{sched} vs fused/kv")


# ------------------------------------------------------------------ full-size workloads (sampled rows)

def _full_size(bwa, orc, name, modes, scheds, per_head, striped=False):
    from ring_exact_attention_amd.inputs import WORKLOADS, make_qkv
    w = WORKLOADS[name]
    log_case(workload=name, stage="inputs", striped=striped)
    q, k, v = make_qkv(w, device="cuda")
    rows = sample_rows(w.B, w.H, w.SQ, w.n, per_head=per_head, seed=w.seed)
    log_case(workload=name, stage="oracle", rows=len(rows))
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    oc = ("striped", w.n) if striped else w.causal
    O, L = orc.attn_fwd(qc, kc, vc, w.scale, causal=oc, rows=rows)
    del qc, kc, vc
    causal = "striped" if striped else w.causal
    for mode in modes:
        for sched in scheds:
            log_case(workload=name, mode=mode, sched=sched)
            o, lse = bwa.bwa_ring_fwd(q, k, v, w.n, sched, mode, causal=causal, scale=w.scale)
            torch.cuda.synchronize()
            o_s = o.reshape(-1, w.D)[torch.as_tensor(rows, device="cuda")]
            l_s = lse.reshape(-1)[torch.as_tensor(rows, device="cuda")]
            check_fwd(o_s, l_s, O, L, w.dtype, f"{name} {mode}/{sched}")
            assert torch.isfinite(o).all() and torch.isfinite(lse).all()


def test_full_lvx_2k_128k(bwa, orc):
    _full_size(bwa, orc, "lvx_2k_128k", MODES, SCHEDS, per_head=6)


def test_full_shortq_256_256k(bwa, orc):
    _full_size(bwa, orc, "shortq_256_256k", ["split", "fused", "rounds"], SCHEDS, per_head=3)


def test_full_causal_64k(bwa, orc):
    _full_size(bwa, orc, "causal_64k", ["fused", "split", "rounds"], SCHEDS, per_head=4)


def test_full_causal_64k_striped(bwa, orc):
    """The causal workload with its rows in the striped order over the 8
    shards (shard w holds positions w, w+8, ...): full size, tiles of 8192
    rows inside one shard, sampled rows against the oracle's striped mask."""
    _full_size(bwa, orc, "causal_64k", ["fused", "split"], ["kv"], per_head=3, striped=True)


@pytest.mark.parametrize("sched", SCHEDS)
def test_merge_partials_vs_oracle(bwa, orc, sched):
    """Oracle partials of each KV shard, merged on the GPU in every query
    block's ring order, equal unblocked attention."""
    B, H, SQ, SKV, D, n = 1, 2, 37, 300, 128, 5
    q, k, v = gen(B, H, SQ, SKV, D, torch.float32, seed=21)
    O, L = orc.attn_fwd(q, k, v, 0.1)
    parts = [orc.attn_partial(q, k, v, 0.1, False, 0, SQ, a, b) for a, b in orc.shard_bounds(SKV, n)]
    op = torch.tensor(np.stack([p[0] for p in parts]), dtype=torch.float32, device="cuda")
    lp = torch.tensor(np.stack([p[1] for p in parts]), dtype=torch.float32, device="cuda")
    o, lse = bwa.bwa_merge_partials(op, lp, n, sched)
    torch.cuda.synchronize()
    check_fwd(o, lse, O, L, "f32", f"merge_partials {sched}")


def test_split_workspace_merge_matches_ring(bwa):
    q, k, v = (x.cuda() for x in gen(1, 2, 300, 2000, 128, torch.bfloat16, seed=22))
    from ring_exact_attention_amd._bwa import split_workspace_views
    ws = torch.empty(bwa.ring_fwd_workspace(q, k, 4, "split"), dtype=torch.uint8, device="cuda")
    o, lse = bwa.bwa_ring_fwd(q, k, v, 4, "q", "split", workspace=ws)
    op, lp = split_workspace_views(ws, 4, 1, 2, 300, 128)
    o2, lse2 = bwa.bwa_merge_partials(op, lp, 4, "q", dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("causal", [False, True])
def test_transfer_mode_is_bitwise_rounds(bwa, causal):
    """The emulated exchange moves the rotating blocks through device copies
    between rounds; the arithmetic is that of ROUNDS, so the results agree bit
    for bit (also with strided [B, S, H, D] inputs)."""
    g = torch.Generator().manual_seed(31 + causal)
    B, H, S, D, n = 1, 3, 700, 128, 5
    base = [(torch.randn(B, S, H, D, generator=g) * 0.5).bfloat16().cuda() for _ in range(3)]
    q, k, v = (t.transpose(1, 2) for t in base)  # strided views
    for sched in SCHEDS:
        log_case(test="transfer", sched=sched, causal=causal)
        o1, l1 = bwa.bwa_ring_fwd(q, k, v, n, sched, "rounds", causal=causal)
        o2, l2 = bwa.bwa_ring_fwd(q, k, v, n, sched, "rounds_transfer", causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), sched


def _stripe_inverse(S, n):
    """Row of the striped layout holding each sequence position (shard w holds
    positions w, w+n, ...), from dealing positions round-robin to shards."""
    shards = [[] for _ in range(n)]
    for t in range(S):
        shards[t % n].append(t)
    pos = np.array([t for sh in shards for t in sh])
    return np.argsort(pos)


@pytest.mark.parametrize("shape", [(1, 2, 512, 128, 4), (1, 1, 384, 64, 3), (2, 2, 1024, 128, 8)],
                         ids=lambda s: "x".join(map(str, s)))
def test_striped_causal_all_modes(bwa, orc, shape):
    """Rows in the striped order (shard w holds positions w, w+n, ...): every
    mode and schedule against the oracle's causal attention on the sequence."""
    B, H, S, D, n = shape
    g = torch.Generator().manual_seed(S + n)
    q, k, v = [(torch.randn(B, H, S, D, generator=g) * 0.5).bfloat16() for _ in range(3)]
    scale = 1.0 / math.sqrt(D)
    O, L = orc.attn_fwd(q, k, v, scale, causal=("striped", n))
    inv = _stripe_inverse(S, n)
    On, Ln = orc.attn_fwd(q[:, :, inv], k[:, :, inv], v[:, :, inv], scale, causal=True)
    np.testing.assert_allclose(O[:, :, inv], On, rtol=1e-12, atol=1e-13)  # oracle self-check
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    for mode in MODES:
        for sched in SCHEDS:
            log_case(test="striped", shape=shape, mode=mode, sched=sched)
            o, lse = bwa.bwa_ring_fwd(qd, kd, vd, n, sched, mode, causal="striped", scale=scale)
            torch.cuda.synchronize()
            check_fwd(o, lse, O, L, "bf16", f"striped {shape} {mode} {sched}")


def test_striped_causal_f32(bwa, orc):
    B, H, S, D, n = 1, 1, 96, 64, 4
    g = torch.Generator().manual_seed(5)
    q, k, v = [torch.randn(B, H, S, D, generator=g) for _ in range(3)]
    O, L = orc.attn_fwd(q, k, v, 0.125, causal=("striped", n))
    for mode in MODES:
        log_case(test="striped f32", mode=mode)
        o, lse = bwa.bwa_ring_fwd(q.cuda(), k.cuda(), v.cuda(), n, "kv", mode, causal="striped",
                                  scale=0.125)
        torch.cuda.synchronize()
        check_fwd(o, lse, O, L, "f32", f"striped f32 {mode}")
