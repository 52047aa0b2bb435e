"""GPU backward and K/V-recompute parity vs the fp64 oracle (through the C ABI)."""
import math

import numpy as np
import pytest
import torch

from tests.parity import check_grad, dq_row_allowance, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bwa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_exact_attention_amd as m
    m.lib()
    return m


def log_case(**kw):
    print("case:", " ".join(f"{a}={b}" for a, b in kw.items()), flush=True)


def gen(B, H, SQ, SKV, D, seed, std=0.5):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(B, H, SQ, D, generator=g) * std).bfloat16()
    k = (torch.randn(B, H, SKV, D, generator=g) * std).bfloat16()
    v = (torch.randn(B, H, SKV, D, generator=g) * std).bfloat16()
    do = torch.randn(B, H, SQ, D, generator=g).bfloat16()
    return q, k, v, do


BWD_SHAPES = [
    # B, H, SQ, SKV, n, causal, D
    (1, 2, 256, 1024, 4, False, 128),
    (1, 2, 300, 1000, 4, False, 128),    # ragged tiles and shards
    (2, 1, 65, 130, 3, False, 128),
    (1, 1, 5, 100, 8, False, 128),       # empty query blocks
    (1, 2, 512, 512, 4, True, 128),
    (1, 1, 300, 300, 3, True, 128),
    (1, 2, 300, 1000, 4, False, 64),     # D = 64
    (2, 1, 65, 130, 3, False, 64),
    (1, 2, 512, 512, 4, True, 64),
    (1, 1, 300, 300, 3, True, 64),
    # rows in the striped order over the n shards (n divides S)
    (1, 2, 512, 512, 4, "striped", 128),
    (1, 1, 384, 384, 3, "striped", 128),  # shards of 128: key tiles end on shard ends
    (1, 1, 300, 300, 5, "striped", 128),  # shards of 60: ragged tiles inside each shard
    (2, 1, 1024, 1024, 8, "striped", 128),
    (1, 2, 384, 384, 3, "striped", 64),
    # at least 8 heads: the fused dK/dV grid is laid out head by head
    (2, 4, 300, 1000, 4, False, 128),
    (1, 8, 384, 384, 3, True, 64),
    (1, 8, 256, 256, 2, "striped", 128),
]


@pytest.mark.parametrize("shape", BWD_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_small(bwa, orc, shape):
    B, H, SQ, SKV, n, causal, D = shape
    scale = 1 / math.sqrt(D)
    q, k, v, do = gen(B, H, SQ, SKV, D, seed=SQ + SKV + D)
    oc = ("striped", n) if causal == "striped" else causal
    ref = orc.attn_bwd(q, k, v, do, scale, oc)
    extra = dq_row_allowance(orc, q, k, v, do, scale, oc)
    qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
    o, lse = bwa.bwa_ring_fwd(qd, kd, vd, n, "kv", "fused", causal=causal, scale=scale)
    for mode in ("fused", "rounds"):
        for sched in ("kv", "q"):
            log_case(shape=shape, mode=mode, sched=sched)
            dq, dk, dv = bwa.bwa_ring_bwd(qd, kd, vd, o, lse, dod, n, sched, mode, causal=causal,
                                          scale=scale)
            torch.cuda.synchronize()
            check_grad(dq.reshape(B * H, SQ, D), ref["dq"], f"dq {shape} {mode}/{sched}",
                       row_extra=extra)
            check_grad(dk.reshape(B * H, SKV, D), ref["dk"], f"dk {shape} {mode}/{sched}")
            check_grad(dv.reshape(B * H, SKV, D), ref["dv"], f"dv {shape} {mode}/{sched}")


@pytest.mark.parametrize("shape", [(2, 3, 130, 700, 4, False, 128), (1, 2, 300, 300, 3, True, 128),
                                   (2, 2, 200, 450, 3, False, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_bwd_strided_layouts_and_guard_bands(bwa, orc, shape):
    """Every input and gradient in [B, S, H, D] storage viewed as [B, H, S, D];
    each gradient written into the middle of a NaN-filled buffer, whose rest
    must stay untouched."""
    B, H, SQ, SKV, n, causal, D = shape
    scale = 1 / math.sqrt(D)
    q, k, v, do = gen(B, H, SQ, SKV, D, seed=SQ * 7 + SKV + D)
    ref = orc.attn_bwd(q, k, v, do, scale, causal)
    extra = dq_row_allowance(orc, q, k, v, do, scale, causal)
    bshd = lambda t: t.transpose(1, 2).contiguous().cuda().transpose(1, 2)
    qs, ks, vs, dos = bshd(q), bshd(k), bshd(v), bshd(do)
    o, lse = bwa.bwa_ring_fwd(q.cuda(), k.cuda(), v.cuda(), n, "kv", "fused", causal=causal,
                              scale=scale)
    os_ = bshd(o.cpu())

    def guarded(S):
        big = torch.full((B, S + 8, H, D + 64), float("nan"), dtype=torch.bfloat16, device="cuda")
        return big, big[:, 4:4 + S, :, 32:32 + D].transpose(1, 2)

    for mode in ("fused", "rounds"):
        for sched in ("kv", "q"):
            log_case(strided=shape, mode=mode, sched=sched)
            (bq, gq), (bk, gk), (bv, gv) = guarded(SQ), guarded(SKV), guarded(SKV)
            bwa.bwa_ring_bwd(qs, ks, vs, os_, lse, dos, n, sched, mode, causal=causal, scale=scale,
                             dq=gq, dk=gk, dv=gv)
            torch.cuda.synchronize()
            for big, g, name, S in ((bq, gq, "dq", SQ), (bk, gk, "dk", SKV), (bv, gv, "dv", SKV)):
                check_grad(g.reshape(B * H, S, D), ref[name], f"{name} strided {shape} {mode}/{sched}",
                           row_extra=extra if name == "dq" else None)
                mask = torch.ones_like(big, dtype=torch.bool)
                mask[:, 4:4 + S, :, 32:32 + D] = False
                assert torch.isnan(big[mask].float()).all(), f"{name}: write outside the view"


def test_bwd_deterministic(bwa):
    q, k, v, do = (x.cuda() for x in gen(1, 2, 512, 4096, 128, seed=1))
    o, lse = bwa.bwa_ring_fwd(q, k, v, 8)
    for mode in ("fused", "rounds"):
        a = bwa.bwa_ring_bwd(q, k, v, o, lse, do, 8, "kv", mode)
        b = bwa.bwa_ring_bwd(q, k, v, o, lse, do, 8, "kv", mode)
        torch.cuda.synchronize()
        for x, y in zip(a, b):
            assert torch.equal(x, y), mode


def test_kv_recompute_small(bwa, orc):
    for (B, S, E, H, D) in [(2, 300, 128, 2, 128), (1, 1000, 256, 3, 128), (1, 64, 64, 2, 64)]:
        g = torch.Generator().manual_seed(S)
        y = (torch.randn(B, S, E, generator=g) * 0.5).bfloat16()
        wk = (torch.randn(H * D, E, generator=g) * 0.1).bfloat16()
        wv = (torch.randn(H * D, E, generator=g) * 0.1).bfloat16()
        log_case(recompute=(B, S, E, H, D))
        k, v = bwa.bwa_kv_recompute(y.cuda(), wk.cuda(), wv.cuda(), H, D)
        torch.cuda.synchronize()
        for got, w in ((k, wk), (v, wv)):
            ref = orc.kv_proj(y, w, H, D)
            err = np.abs(to64(got) - ref)
            # one bf16 rounding of the fp32 accumulator: half an ulp, <= 2^-8 relative
            assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 1e-6), err.max()


def test_kv_recompute_repeatable(bwa):
    """The K/V GEMM at the recompute workload's full shape, run six times on the
    same inputs, gives bitwise the same K and V: every output element is one fp32
    sum in a fixed order, so any difference is a read of an LDS stage that another
    wave has already overwritten (the double-buffered stages share one barrier)."""
    from ring_exact_attention_amd.inputs import WORKLOADS, make_recompute
    w = WORKLOADS["recompute_bwd"]
    log_case(workload=w.name, stage="repeated K/V GEMM")
    y, wk, wv = make_recompute(w, device="cuda")
    k0, v0 = bwa.bwa_kv_recompute(y, wk, wv, w.H, w.D)
    k, v = torch.empty_like(k0), torch.empty_like(v0)
    for _ in range(5):
        bwa.bwa_kv_recompute(y, wk, wv, w.H, w.D, k=k, v=v)
        torch.cuda.synchronize()
        assert torch.equal(k, k0) and torch.equal(v, v0)


def test_kv_recompute_bwd_repeatable(bwa):
    """dW_k^T, dW_v^T and dy at 16384 keys, E = 4096, 32 heads of 128, run three
    times: bitwise the same results (fixed-order fp32 sums; a difference would be
    an LDS stage read after another wave overwrote it)."""
    B, S, E, H, D = 1, 16384, 4096, 32, 128
    g = torch.Generator(device="cuda").manual_seed(11)
    y = (torch.randn(B, S, E, device="cuda", generator=g) * 0.02).bfloat16()
    wk = (torch.randn(H * D, E, device="cuda", generator=g) * 0.02).bfloat16()
    wv = (torch.randn(H * D, E, device="cuda", generator=g) * 0.02).bfloat16()
    dk = torch.randn(B, H, S, D, device="cuda", generator=g).bfloat16()
    dv = torch.randn(B, H, S, D, device="cuda", generator=g).bfloat16()
    log_case(stage="repeated gradient GEMMs", shape=(B, S, E, H, D))
    ref = [t.clone() for t in bwa.bwa_kv_recompute_bwd(y, wk, wv, dk, dv)]
    for _ in range(2):
        got = bwa.bwa_kv_recompute_bwd(y, wk, wv, dk, dv)
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(got, ref))


def test_kv_recompute_strided_output(bwa, orc):
    """Write K into a [B, S, H, D] buffer through strides."""
    B, S, E, H, D = 1, 200, 128, 2, 128
    g = torch.Generator().manual_seed(4)
    y = (torch.randn(B, S, E, generator=g) * 0.5).bfloat16()
    w = (torch.randn(H * D, E, generator=g) * 0.1).bfloat16()
    kb = torch.zeros(B, S, H, D, dtype=torch.bfloat16, device="cuda")
    vb = torch.zeros(B, H, S, D, dtype=torch.bfloat16, device="cuda")
    bwa.bwa_kv_recompute(y.cuda(), w.cuda(), w.cuda(), H, D, k=kb.transpose(1, 2), v=vb)
    torch.cuda.synchronize()
    ref = orc.kv_proj(y, w, H, D)
    assert np.abs(to64(kb.transpose(1, 2)) - ref).max() <= 2.0 ** -8 * np.abs(ref).max()
    assert torch.equal(kb.transpose(1, 2), vb)


def test_full_recompute_bwd(bwa, orc):
    """Recompute + backward workload: y [1, 65536, 4096], W_k, W_v [4096, 4096],
    32 heads, S_Q = 2048, n = 8.  Checks sampled K/V rows of the GEMM against the
    exact fp64 projection, and dQ/dK/dV of two full heads against the oracle's
    exact gradients computed from the exact (fp64) K and V."""
    from ring_exact_attention_amd.inputs import WORKLOADS, make_dout, make_qkv, make_recompute
    w = WORKLOADS["recompute_bwd"]
    log_case(workload=w.name, stage="inputs")
    y, wk, wv = make_recompute(w, device="cuda")
    q, _, _ = make_qkv(w.resized(SKV=1), device="cuda")
    do = make_dout(w, device="cuda")
    k, v = bwa.bwa_kv_recompute(y, wk, wv, w.H, w.D)
    o, lse = bwa.bwa_ring_fwd(q, k, v, w.n, "kv", "fused", scale=w.scale)
    grads = {}
    for sched, mode in (("kv", "fused"), ("q", "fused"), ("kv", "rounds"), ("q", "rounds")):
        log_case(workload=w.name, stage="backward", sched=sched, mode=mode)
        dq, dk, dv = bwa.bwa_ring_bwd(q, k, v, o, lse, do, w.n, sched, mode, scale=w.scale)
        torch.cuda.synchronize()
        for x in (dq, dk, dv):
            assert torch.isfinite(x).all()
        grads[(sched, mode)] = (dq, dk, dv)
    for x in (k, v, o):
        assert torch.isfinite(x).all()

    yc, wkc, wvc = y.cpu(), wk.cpu(), wv.cpu()
    g = np.random.default_rng(w.seed)
    rows = np.sort(g.choice(w.SKV, size=64, replace=False))
    log_case(workload=w.name, stage="oracle projection rows")
    for got, wt in ((k, wkc), (v, wvc)):
        ref = orc.kv_proj(yc, wt, w.H, w.D, rows=rows).reshape(len(rows), w.H, w.D)
        gs = to64(got[0, :, torch.as_tensor(rows, device="cuda")].permute(1, 0, 2))
        assert np.all(np.abs(gs - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)

    heads = [0, 17]
    log_case(workload=w.name, stage="oracle exact K, V of two heads")
    K = np.stack([orc.kv_proj(yc, wkc[h * w.D:(h + 1) * w.D], 1, w.D)[0, 0] for h in heads])[None]
    V = np.stack([orc.kv_proj(yc, wvc[h * w.D:(h + 1) * w.D], 1, w.D)[0, 0] for h in heads])[None]
    qh = q[:, heads].cpu().double().numpy()
    doh = do[:, heads].cpu().double().numpy()
    keys = np.sort(g.choice(w.SKV, size=256, replace=False))
    log_case(workload=w.name, stage="oracle backward")
    ref = orc.attn_bwd(qh, K, V, doh, w.scale, keys=keys)
    kk = torch.as_tensor(keys, device="cuda")
    for (sched, mode), (dq, dk, dv) in grads.items():
        tag = f"{sched}/{mode}"
        check_grad(dq[0, heads], ref["dq"], f"dq full {tag}")
        check_grad(dk[0, heads][:, kk], ref["dk"], f"dk full {tag} (sampled keys)")
        check_grad(dv[0, heads][:, kk], ref["dv"], f"dv full {tag} (sampled keys)")


# ---------------------------------------------------------------- gradients through the recompute

def _check_rows(got, ref, what, rel=2e-5):
    """fp32 accumulation of exact bf16 products: every element within `rel` of
    the largest reference magnitude of its row block."""
    got = np.asarray(got, np.float64)
    err = np.abs(got - ref).max()
    scale = np.abs(ref).max()
    assert err <= rel * scale, f"{what}: max err {err:.3e} vs max |ref| {scale:.3e}"
    assert np.linalg.norm(got - ref) <= rel * np.linalg.norm(ref), what


@pytest.mark.parametrize("shape", [(1, 64, 256, 2, 128), (2, 128, 256, 4, 64),
                                   (1, 320, 512, 2, 128)], ids=lambda s: "x".join(map(str, s)))
def test_kv_recompute_bwd_small(bwa, orc, shape):
    B, S, E, H, D = shape
    g = torch.Generator().manual_seed(S + E)
    y = (torch.randn(B, S, E, generator=g) * 0.5).bfloat16()
    wk = (torch.randn(H * D, E, generator=g) * 0.1).bfloat16()
    wv = (torch.randn(H * D, E, generator=g) * 0.1).bfloat16()
    gk = torch.randn(B, H, S, D, generator=g).bfloat16()
    gv = torch.randn(B, H, S, D, generator=g).bfloat16()
    log_case(recompute_bwd=shape)
    dwk, dwv, dy = bwa.bwa_kv_recompute_bwd(y.cuda(), wk.cuda(), wv.cuda(), gk.cuda(), gv.cuda())
    torch.cuda.synchronize()
    _check_rows(dwk.cpu().numpy(), orc.kv_grad_w(y, gk), "dW_k")
    _check_rows(dwv.cpu().numpy(), orc.kv_grad_w(y, gv), "dW_v")
    _check_rows(dy.cpu().numpy().reshape(B * S, E), orc.kv_grad_y(gk, gv, wk, wv), "dy")


def test_kv_recompute_bwd_accumulate_strided_and_partial_outputs(bwa, orc):
    B, S, E, H, D = 1, 128, 256, 2, 128
    g = torch.Generator().manual_seed(77)
    y = (torch.randn(B, S, E, generator=g) * 0.5).bfloat16().cuda()
    wk = (torch.randn(H * D, E, generator=g) * 0.1).bfloat16().cuda()
    wv = (torch.randn(H * D, E, generator=g) * 0.1).bfloat16().cuda()
    # dK, dV stored [B, S, H, D] and passed as [B, H, S, D] views (equal strides)
    gk = torch.randn(B, S, H, D, generator=g).bfloat16().cuda().transpose(1, 2)
    gv = torch.randn(B, S, H, D, generator=g).bfloat16().cuda().transpose(1, 2)
    log_case(recompute_bwd="strided+accumulate")
    ref_w = orc.kv_grad_w(y.cpu(), gk.cpu().contiguous())
    ref_y = orc.kv_grad_y(gk.cpu().contiguous(), gv.cpu().contiguous(), wk.cpu(), wv.cpu())
    dwk = torch.full((H * D, E), 0.25, device="cuda")
    dy = torch.full((B, S, E), -0.5, device="cuda")
    bwa.bwa_kv_recompute_bwd(y, wk, wv, gk, gv, dwk_t=dwk, dy=dy, accumulate=True,
                             outputs=("dwk_t", "dy"))
    bwa.bwa_kv_recompute_bwd(y, wk, wv, gk, gv, dwk_t=dwk, dy=dy, accumulate=True,
                             outputs=("dwk_t", "dy"))
    torch.cuda.synchronize()
    _check_rows(dwk.cpu().numpy() - 0.25, 2 * ref_w, "dW_k accumulated twice")
    _check_rows(dy.cpu().numpy().reshape(B * S, E) + 0.5, 2 * ref_y, "dy accumulated twice")
    only_dy = bwa.bwa_kv_recompute_bwd(y, wk, wv, gk, gv, outputs=("dy",))
    torch.cuda.synchronize()
    assert only_dy[0] is None and only_dy[1] is None
    _check_rows(only_dy[2].cpu().numpy().reshape(B * S, E), ref_y, "dy alone")


def test_kv_recompute_bwd_full_size_sampled(bwa, orc):
    """Recompute workload sizes (y [1, 65536, 4096], W [4096, 4096], 32 heads of
    128): sampled rows of dW_k, dW_v (each a 65536-term sum) and of dy."""
    from ring_exact_attention_amd.inputs import WORKLOADS, make_recompute
    w = WORKLOADS["recompute_bwd"]
    log_case(workload=w.name, stage="weight and feature gradients")
    y, wk, wv = make_recompute(w, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(w.seed + 303)
    gk = torch.randn(w.B, w.H, w.SKV, w.D, generator=g, device="cuda").bfloat16()
    gv = torch.randn(w.B, w.H, w.SKV, w.D, generator=g, device="cuda").bfloat16()
    dwk, dwv, dy = bwa.bwa_kv_recompute_bwd(y, wk, wv, gk, gv)
    torch.cuda.synchronize()
    for x in (dwk, dwv, dy):
        assert torch.isfinite(x).all()
    yc, gkc, gvc = y.cpu(), gk.cpu(), gv.cpu()
    nrows = [0, 1234, w.H * w.D - 1]
    log_case(workload=w.name, stage="oracle dW rows")
    _check_rows(dwk[nrows].cpu().numpy(), orc.kv_grad_w(yc, gkc, rows=nrows), "dW_k rows", 1e-4)
    _check_rows(dwv[nrows].cpu().numpy(), orc.kv_grad_w(yc, gvc, rows=nrows), "dW_v rows", 1e-4)
    srows = [0, 40000, w.B * w.SKV - 1]
    log_case(workload=w.name, stage="oracle dy rows")
    ref = orc.kv_grad_y(gkc, gvc, wk.cpu(), wv.cpu(), rows=srows)
    _check_rows(dy.reshape(-1, w.E)[srows].cpu().numpy(), ref, "dy rows", 1e-4)
