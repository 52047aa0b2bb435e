"""Pins for the fp64 CPU oracle, against things other than itself.

The pages print no worked numeric example, so every pin is a brute-force
evaluation, a closed form, an invariant the method must satisfy, or an
independent library routine (PyTorch's scaled_dot_product_attention -- the
check the LV-XAttn review says the paper's forward was validated against --
torch autograd, scipy's logsumexp, numpy matmul).
"""
import itertools
import math

import numpy as np
import pytest
import torch
from scipy.special import logsumexp


def rnd(shape, seed, std=1.0):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape) * std


def brute_force(q, k, v, tau, causal):
    """Pure-Python softmax without max shift; fsum for the sums."""
    B, H, SQ, D = q.shape
    SKV = k.shape[2]
    O = np.zeros((B, H, SQ, D))
    L = np.zeros((B, H, SQ))
    for b in range(B):
        for h in range(H):
            for i in range(SQ):
                js = [j for j in range(SKV) if (not causal or j <= i)]
                e = {j: math.exp(tau * math.fsum(q[b, h, i, d] * k[b, h, j, d] for d in range(D)))
                     for j in js}
                z = math.fsum(e.values())
                L[b, h, i] = math.log(z)
                for d in range(D):
                    O[b, h, i, d] = math.fsum(e[j] * v[b, h, j, d] for j in js) / z
    return O, L


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape", [(1, 1, 1, 1, 1), (2, 2, 3, 7, 4), (1, 2, 4, 9, 3)])
def test_forward_brute_force(orc, shape, causal):
    B, H, SQ, SKV, D = shape
    if causal:
        SKV = SQ
    q, k, v = rnd((B, H, SQ, D), 1), rnd((B, H, SKV, D), 2), rnd((B, H, SKV, D), 3)
    tau = 1 / math.sqrt(D)
    O, L = orc.attn_fwd(q, k, v, tau, causal)
    Ob, Lb = brute_force(q, k, v, tau, causal)
    np.testing.assert_allclose(O, Ob, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(L, Lb, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_forward_vs_torch_sdpa(orc, D, causal):
    SQ, SKV = (40, 40) if causal else (24, 300)
    q = torch.randn(2, 3, SQ, D, dtype=torch.float64, generator=torch.Generator().manual_seed(5))
    k = torch.randn(2, 3, SKV, D, dtype=torch.float64, generator=torch.Generator().manual_seed(6))
    v = torch.randn(2, 3, SKV, D, dtype=torch.float64, generator=torch.Generator().manual_seed(7))
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal)
    O, L = orc.attn_fwd(q.numpy(), k.numpy(), v.numpy(), 1 / math.sqrt(D), causal)
    np.testing.assert_allclose(O, ref.numpy(), rtol=1e-11, atol=1e-12)
    s = np.einsum("bhid,bhjd->bhij", q.numpy(), k.numpy()) / math.sqrt(D)
    if causal:
        s = np.where(np.tril(np.ones((SQ, SKV), bool)), s, -np.inf)
    np.testing.assert_allclose(L, logsumexp(s, axis=-1), rtol=1e-12, atol=1e-12)


def test_forward_rows_subset_matches_full(orc):
    q, k, v = rnd((2, 2, 10, 8), 11), rnd((2, 2, 33, 8), 12), rnd((2, 2, 33, 8), 13)
    O, L = orc.attn_fwd(q, k, v, 0.3)
    rows = [0, 7, 19, 20, 39]
    Os, Ls = orc.attn_fwd(q, k, v, 0.3, rows=rows)
    np.testing.assert_array_equal(Os, O.reshape(-1, 8)[rows])
    np.testing.assert_array_equal(Ls, L.reshape(-1)[rows])


def test_bf16_inputs_read_exactly(orc):
    g = torch.Generator().manual_seed(3)
    q = (torch.randn(1, 2, 6, 16, generator=g) * 0.5).bfloat16()
    k = (torch.randn(1, 2, 50, 16, generator=g) * 0.5).bfloat16()
    v = torch.randn(1, 2, 50, 16, generator=g).bfloat16()
    O, L = orc.attn_fwd(q, k, v, 0.25)
    O2, L2 = orc.attn_fwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), 0.25)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(L, L2)
    O3, L3 = orc.attn_fwd(q.float().numpy(), k.float().numpy(), v.float().numpy(), 0.25)
    np.testing.assert_array_equal(O, O3)


# ---------------------------------------------------------------- closed forms

def test_zero_query_gives_mean_of_values(orc):
    SKV = 37
    q = np.zeros((1, 2, 5, 8))
    k, v = rnd((1, 2, SKV, 8), 21), rnd((1, 2, SKV, 8), 22)
    O, L = orc.attn_fwd(q, k, v, 0.35)
    np.testing.assert_allclose(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape),
                               rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(L, math.log(SKV), rtol=1e-15)


def test_equal_keys_give_uniform_weights(orc):
    q = rnd((1, 1, 4, 8), 23)
    k = np.broadcast_to(rnd((1, 1, 1, 8), 24), (1, 1, 19, 8)).copy()
    v = rnd((1, 1, 19, 8), 25)
    O, L = orc.attn_fwd(q, k, v, 0.5)
    np.testing.assert_allclose(O, np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape),
                               rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(L[0, 0], 0.5 * (q[0, 0] @ k[0, 0, 0]) + math.log(19), rtol=1e-13)


def test_single_key(orc):
    q, k, v = rnd((2, 1, 3, 4), 26), rnd((2, 1, 1, 4), 27), rnd((2, 1, 1, 4), 28)
    O, L = orc.attn_fwd(q, k, v, 0.7)
    np.testing.assert_allclose(O, np.broadcast_to(v, O.shape), rtol=1e-15)
    np.testing.assert_allclose(L, 0.7 * np.einsum("bhid,bhd->bhi", q, k[:, :, 0]), rtol=1e-14)


def test_causal_first_row(orc):
    q, k, v = rnd((1, 2, 9, 4), 29), rnd((1, 2, 9, 4), 30), rnd((1, 2, 9, 4), 31)
    O, L = orc.attn_fwd(q, k, v, 0.5, causal=True)
    np.testing.assert_allclose(O[:, :, 0], v[:, :, 0], rtol=1e-15)
    np.testing.assert_allclose(L[:, :, 0], 0.5 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                               rtol=1e-14)


def test_one_hot_dominant_key(orc):
    SKV, D, jstar = 50, 8, 17
    q = rnd((1, 1, 1, D), 32)
    k = rnd((1, 1, SKV, D), 33) * 0.01
    v = rnd((1, 1, SKV, D), 34)
    c = 200.0 / float(q[0, 0, 0] @ q[0, 0, 0])
    k[0, 0, jstar] = c * q[0, 0, 0]
    tau = 1.0
    s = tau * (k[0, 0] @ q[0, 0, 0])
    margin = s[jstar] - np.max(np.delete(s, jstar))
    assert margin >= 40
    O, _ = orc.attn_fwd(q, k, v, tau)
    bound = (SKV - 1) * math.exp(-margin) * np.abs(v).max() * 2
    assert np.abs(O[0, 0, 0] - v[0, 0, jstar]).max() <= bound + 1e-15


def test_shift_invariance(orc):
    q, k, v = rnd((1, 2, 6, 8), 35), rnd((1, 2, 21, 8), 36), rnd((1, 2, 21, 8), 37)
    tau = 0.4
    c = rnd((8,), 38)
    O, L = orc.attn_fwd(q, k, v, tau)
    O2, L2 = orc.attn_fwd(q, k + c, v, tau)
    np.testing.assert_allclose(O2, O, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(L2, L + tau * np.einsum("bhid,d->bhi", q, c), rtol=1e-12)
    O3, L3 = orc.attn_fwd(q, k, v + 2.5, tau)
    np.testing.assert_allclose(O3, O + 2.5, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(L3, L, rtol=0, atol=0)


def test_key_permutation_invariance(orc):
    q, k, v = rnd((1, 1, 5, 8), 39), rnd((1, 1, 30, 8), 40), rnd((1, 1, 30, 8), 41)
    perm = np.random.default_rng(42).permutation(30)
    O, L = orc.attn_fwd(q, k, v, 0.3)
    O2, L2 = orc.attn_fwd(q, k[:, :, perm], v[:, :, perm], 0.3)
    np.testing.assert_allclose(O2, O, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(L2, L, rtol=1e-13)


# ---------------------------------------------------------------- merge

def test_merge_identity_and_empty(orc):
    o, l = rnd((4, 8), 50), rnd((4,), 51)
    z, ninf = np.zeros((4, 8)), np.full((4,), -np.inf)
    for a, b in [((o, l), (z, ninf)), ((z, ninf), (o, l))]:
        O, L = orc.merge(*a, *b)
        np.testing.assert_array_equal(O, o)
        np.testing.assert_array_equal(L, l)
    O, L = orc.merge(z, ninf, z, ninf)
    assert np.all(O == 0) and np.all(L == -np.inf)


def test_merge_commutative_associative(orc):
    p = [(rnd((6, 8), 60 + i), rnd((6,), 70 + i) * 3) for i in range(3)]
    ab = orc.merge(*p[0], *p[1])
    ba = orc.merge(*p[1], *p[0])
    np.testing.assert_allclose(ab[0], ba[0], rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(ab[1], ba[1], rtol=1e-15)
    left = orc.merge(*ab, *p[2])
    right = orc.merge(*p[0], *orc.merge(*p[1], *p[2]))
    np.testing.assert_allclose(left[0], right[0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(left[1], right[1], rtol=1e-14)


def test_merge_extreme_lse_no_nan(orc):
    oa, ob = rnd((3, 4), 80), rnd((3, 4), 81)
    la = np.array([1000.0, -1000.0, 0.0])
    lb = np.array([-1000.0, 1000.0, -np.inf])
    O, L = orc.merge(oa, la, ob, lb)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    np.testing.assert_allclose(O[0], oa[0])
    np.testing.assert_allclose(O[1], ob[1])
    np.testing.assert_allclose(O[2], oa[2])


def _splits(S, n):
    for cuts in itertools.combinations(range(1, S), n - 1):
        b = (0,) + cuts + (S,)
        yield [(b[i], b[i + 1]) for i in range(n)]


def test_every_split_and_order_equals_unblocked(orc):
    """S_KV = 12: every contiguous split into n <= 4 blocks, every merge order."""
    SKV, D = 12, 4
    q, k, v = rnd((1, 2, 3, D), 90), rnd((1, 2, SKV, D), 91), rnd((1, 2, SKV, D), 92)
    tau = 0.5
    O, L = orc.attn_fwd(q, k, v, tau)
    count = 0
    for n in range(1, 5):
        for split in _splits(SKV, n):
            parts = [orc.attn_partial(q, k, v, tau, False, 0, 3, a, b) for a, b in split]
            for order in itertools.permutations(range(n)):
                Oa = np.zeros_like(O)
                La = np.full_like(L, -np.inf)
                for t in order:
                    Oa, La = orc.merge(Oa, La, *parts[t])
                np.testing.assert_allclose(Oa, O, rtol=1e-13, atol=1e-14)
                np.testing.assert_allclose(La, L, rtol=1e-13, atol=1e-14)
                count += 1
    assert count == 1 + 11 * 2 + 55 * 6 + 165 * 24


def test_random_noncontiguous_partitions(orc):
    SKV = 40
    q, k, v = rnd((1, 1, 4, 8), 93), rnd((1, 1, SKV, 8), 94), rnd((1, 1, SKV, 8), 95)
    O, L = orc.attn_fwd(q, k, v, 0.4)
    g = np.random.default_rng(96)
    for _ in range(5):
        perm = g.permutation(SKV)
        kp, vp = k[:, :, perm], v[:, :, perm]
        cuts = np.sort(g.choice(np.arange(1, SKV), size=4, replace=False))
        bounds = [0, *cuts.tolist(), SKV]
        Oa, La = np.zeros_like(O), np.full_like(L, -np.inf)
        for a, b in zip(bounds[:-1], bounds[1:]):
            Oa, La = orc.merge(Oa, La, *orc.attn_partial(q, kp, vp, 0.4, False, 0, 4, a, b))
        np.testing.assert_allclose(Oa, O, rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(La, L, rtol=1e-13)


def test_partial_of_empty_range_is_identity(orc):
    q, k, v = rnd((1, 1, 3, 4), 97), rnd((1, 1, 8, 4), 98), rnd((1, 1, 8, 4), 99)
    O, L = orc.attn_partial(q, k, v, 0.5, False, 0, 3, 5, 5)
    assert np.all(O == 0) and np.all(L == -np.inf)


# ---------------------------------------------------------------- schedules

@pytest.mark.parametrize("sched", [0, 1])
@pytest.mark.parametrize("n", range(1, 9))
def test_rounds_are_perfect_matchings(orc, n, sched):
    seen = set()
    for r in range(n):
        pairs = [orc.ring_pair(sched, n, r, w) for w in range(n)]
        assert sorted(p[0] for p in pairs) == list(range(n))
        assert sorted(p[1] for p in pairs) == list(range(n))
        seen.update(pairs)
    assert seen == {(a, b) for a in range(n) for b in range(n)}


def test_schedule_directions():
    """KV-stationary: the query block moves to worker w+1 each round (worker w
    receives from w-1); Q-stationary: the KV shard moves the same way."""
    import oracle
    n = 5
    for w in range(n):
        assert oracle.ring_pair(0, n, 0, w) == (w, w)
        assert oracle.ring_pair(1, n, 0, w) == (w, w)
        assert oracle.ring_pair(0, n, 1, w) == ((w - 1) % n, w)
        assert oracle.ring_pair(1, n, 1, w) == (w, (w - 1) % n)
        # what worker w holds in round r + 1 is what worker w - 1 held in round r
        for r in range(n - 1):
            assert oracle.ring_pair(0, n, r + 1, w)[0] == oracle.ring_pair(0, n, r, (w - 1) % n)[0]
            assert oracle.ring_pair(1, n, r + 1, w)[1] == oracle.ring_pair(1, n, r, (w - 1) % n)[1]


def test_shard_bounds(orc):
    assert orc.shard_bounds(1024, 4) == [(0, 256), (256, 512), (512, 768), (768, 1024)]
    b = orc.shard_bounds(10, 3)
    assert b == [(0, 3), (3, 6), (6, 10)]
    for S in range(1, 30):
        for n in range(1, S + 1):
            bb = orc.shard_bounds(S, n)
            assert bb[0][0] == 0 and bb[-1][1] == S
            assert all(x[1] == y[0] for x, y in zip(bb, bb[1:]))
            assert max(e - s for s, e in bb) - min(e - s for s, e in bb) <= 1


@pytest.mark.parametrize("sched", [0, 1])
@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 8])
def test_ring_forward_equals_unblocked(orc, n, sched):
    q, k, v = rnd((1, 2, 17, 8), 100), rnd((1, 2, 43, 8), 101), rnd((1, 2, 43, 8), 102)
    O, L = orc.attn_fwd(q, k, v, 0.35)
    Or, Lr = orc.ring_fwd(q, k, v, 0.35, n, sched)
    np.testing.assert_allclose(Or, O, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(Lr, L, rtol=1e-13)


@pytest.mark.parametrize("sched", [0, 1])
@pytest.mark.parametrize("n", [1, 2, 4, 7])
def test_ring_forward_causal_equals_unblocked(orc, n, sched):
    S = 29
    q, k, v = rnd((1, 2, S, 8), 103), rnd((1, 2, S, 8), 104), rnd((1, 2, S, 8), 105)
    O, L = orc.attn_fwd(q, k, v, 0.35, causal=True)
    Or, Lr = orc.ring_fwd(q, k, v, 0.35, n, sched, causal=True)
    np.testing.assert_allclose(Or, O, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(Lr, L, rtol=1e-13)


def test_tiny_f32_workload_ring_matches(orc):
    """The tiny fp32 workload (n = 4 blocks of 256) in full."""
    from ring_exact_attention_amd.inputs import WORKLOADS, make_qkv
    w = WORKLOADS["tiny_f32"]
    q, k, v = make_qkv(w)
    O, L = orc.attn_fwd(q, k, v, w.scale)
    for sched in (0, 1):
        Or, Lr = orc.ring_fwd(q, k, v, w.scale, w.n, sched)
        np.testing.assert_allclose(Or, O, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(Lr, L, rtol=1e-13)
    ref = torch.nn.functional.scaled_dot_product_attention(q.double(), k.double(), v.double())
    np.testing.assert_allclose(O, ref.numpy(), rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- backward

def torch_grads(q, k, v, do, tau, causal):
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = qt @ kt.transpose(-1, -2) * tau
    if causal:
        S = s.shape[-1]
        s = s.masked_fill(~torch.ones(S, S, dtype=torch.bool).tril(), float("-inf"))
    o = torch.softmax(s, dim=-1) @ vt
    o.backward(torch.tensor(do))
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy(), o.detach().numpy()


@pytest.mark.parametrize("causal", [False, True])
def test_backward_vs_torch_autograd(orc, causal):
    B, H, SQ, SKV, D = 2, 2, 7, 7 if causal else 23, 8
    q, k, v = rnd((B, H, SQ, D), 110), rnd((B, H, SKV, D), 111), rnd((B, H, SKV, D), 112)
    do = rnd((B, H, SQ, D), 113)
    tau = 0.4
    gq, gk, gv, o = torch_grads(q, k, v, do, tau, causal)
    r = orc.attn_bwd(q, k, v, do, tau, causal)
    np.testing.assert_allclose(r["dq"], gq.reshape(B * H, SQ, D), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(r["dk"], gk.reshape(B * H, SKV, D), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(r["dv"], gv.reshape(B * H, SKV, D), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(r["delta"], np.einsum("bhid,bhid->bhi", do, o).reshape(B * H, SQ),
                               rtol=1e-11, atol=1e-13)


def test_backward_finite_differences(orc):
    B, H, SQ, SKV, D = 1, 1, 3, 5, 3
    q, k, v = rnd((B, H, SQ, D), 120), rnd((B, H, SKV, D), 121), rnd((B, H, SKV, D), 122)
    do = rnd((B, H, SQ, D), 123)
    tau, h = 0.6, 1e-6
    r = orc.attn_bwd(q, k, v, do, tau)

    def loss(qq, kk, vv):
        O, _ = orc.attn_fwd(qq, kk, vv, tau)
        return float(np.sum(O * do))

    for name, x in (("dq", q), ("dk", k), ("dv", v)):
        g = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = [xp if y is x else y for y in (q, k, v)]
            args_m = [xm if y is x else y for y in (q, k, v)]
            g[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        np.testing.assert_allclose(r[name].reshape(x.shape), g, rtol=1e-6, atol=1e-8)


def test_backward_identities(orc):
    B, H, SQ, SKV, D = 1, 2, 9, 31, 8
    q, k, v = rnd((B, H, SQ, D), 130), rnd((B, H, SKV, D), 131), rnd((B, H, SKV, D), 132)
    do = rnd((B, H, SQ, D), 133)
    r = orc.attn_bwd(q, k, v, do, 0.3)
    # each row of dS sums to zero, so the key gradients sum to zero
    np.testing.assert_allclose(r["dk"].sum(axis=1), 0, atol=1e-12)
    # each row of P sums to one
    np.testing.assert_allclose(r["dv"].sum(axis=1), do.reshape(B * H, SQ, D).sum(axis=1),
                               rtol=1e-12, atol=1e-12)
    # linear in dO
    r2 = orc.attn_bwd(q, k, v, 2.0 * do, 0.3)
    r3 = orc.attn_bwd(q, k, v, do + 2.0 * do, 0.3)
    for name in ("dq", "dk", "dv"):
        np.testing.assert_allclose(r2[name], 2 * r[name], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(r3[name], r[name] + r2[name], rtol=1e-12, atol=1e-13)
    # equal value rows make O independent of the logits: dQ = dK = 0
    ve = np.broadcast_to(v[:, :, :1], v.shape).copy()
    r4 = orc.attn_bwd(q, k, ve, do, 0.3)
    np.testing.assert_allclose(r4["dq"], 0, atol=1e-13)
    np.testing.assert_allclose(r4["dk"], 0, atol=1e-13)


def test_backward_subsets_match_full(orc):
    B, H, SQ, SKV, D = 2, 2, 6, 19, 8
    q, k, v = rnd((B, H, SQ, D), 140), rnd((B, H, SKV, D), 141), rnd((B, H, SKV, D), 142)
    do = rnd((B, H, SQ, D), 143)
    full = orc.attn_bwd(q, k, v, do, 0.3)
    sub = orc.attn_bwd(q, k, v, do, 0.3, heads=[3, 1], keys=[0, 18, 5])
    for t, hh in enumerate([3, 1]):
        np.testing.assert_array_equal(sub["dq"][t], full["dq"][hh])
        np.testing.assert_array_equal(sub["dk"][t], full["dk"][hh][[0, 18, 5]])
        np.testing.assert_array_equal(sub["dv"][t], full["dv"][hh][[0, 18, 5]])
    O, L = orc.attn_fwd(q, k, v, 0.3)
    np.testing.assert_allclose(full["lse"], L.reshape(B * H, SQ), rtol=1e-14)


# ---------------------------------------------------------------- projection

def test_projection_vs_numpy(orc):
    B, S, E, H, D = 2, 5, 12, 3, 4
    y = rnd((B, S, E), 150)
    w_t = rnd((H * D, E), 151)
    K = orc.kv_proj(y, w_t, H, D)
    ref = (y @ w_t.T).reshape(B, S, H, D).transpose(0, 2, 1, 3)
    np.testing.assert_allclose(K, ref, rtol=1e-13, atol=1e-14)
    # the (b, s, h, d) element is the dot of y[b, s] with column h*D + d of W
    assert abs(K[1, 2, 3, 1] - float(y[1, 3] @ w_t[2 * D + 1])) < 1e-13
    rows = [0, 9, 4]
    Kr = orc.kv_proj(y, w_t, H, D, rows=rows)
    np.testing.assert_allclose(Kr, (y.reshape(B * S, E) @ w_t.T)[rows], rtol=1e-13, atol=1e-14)
    K2 = orc.kv_proj(2 * y + 1, w_t, H, D)
    K1 = orc.kv_proj(np.ones_like(y), w_t, H, D)
    np.testing.assert_allclose(K2, 2 * K + K1, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- schedule cost model

def test_schedule_model_comm_volume_video_mme(orc):
    """LV-XAttn review, "The paper's central claim": for Llama 3-V on Video-MME
    (S_Q = 5,514, S_KV = 15,279,944) rotating Q, O and the softmax statistics
    instead of K, V cuts communication volume to 0.04% of Ring Attention's."""
    for d in (1024, 4096, 8192):
        for n in (4, 16, 64):
            _, t = orc.schedule_model(5514, 15279944, d, n, 312e12, 25e9)
            ratio = t["comm_kv"] / t["comm_q"]
            assert round(100 * ratio, 2) == 0.04, (d, n, ratio)


def test_schedule_model_speedup_closed_form(orc):
    """When the LV-XAttn round is compute-bound and the Ring round is
    communication-bound, the modelled speedup is n * FLOPS / (S_Q * BW) for
    2-byte elements (the corrected reading of the review's closed form)."""
    for (sq, skv, d, n, fl, bw) in [(3128, 2_000_000, 4096, 16, 312e12, 25e9),
                                    (2048, 1_048_576, 4096, 8, 2.5e15, 153e9),
                                    (512, 400_000, 1024, 4, 1e14, 1e10)]:
        c, t = orc.schedule_model(sq, skv, d, n, fl, bw, elem_bytes=2)
        assert c == "kv"
        assert t["round_kv"] == t["compute"] > t["comm_kv"]
        assert t["round_q"] == t["comm_q"] > t["compute"]
        speedup = t["round_q"] / t["round_kv"]
        assert abs(speedup / (n * fl / (sq * bw)) - 1) < 1e-12


def test_schedule_model_choices(orc):
    # long visual input: KV stays put
    assert orc.schedule_model(5514, 15279944, 4096, 16, 312e12, 25e9)[0] == "kv"
    # S_Q = S_KV, communication-bound: LV-XAttn sends S/n more elements
    c, t = orc.schedule_model(65536, 65536, 4096, 16, 1e18, 1e9)
    assert c == "q" and t["comm_kv"] > t["comm_q"]
    # far more queries than keys: Ring moves the smaller blocks
    assert orc.schedule_model(1_000_000, 4096, 4096, 8, 312e12, 25e9)[0] == "q"
    # both compute-bound: equal rounds, the tie goes to LV-XAttn
    c, t = orc.schedule_model(8192, 8192, 4096, 2, 1e9, 1e18)
    assert c == "kv" and t["round_kv"] == t["round_q"] == t["compute"]
    # compute of one round: two contractions of an (S_Q/n x d) block with an
    # (S_KV/n x d) block, a multiply-add counted as two (brute count below)
    sq, skv, d, n = 6, 10, 3, 2
    madds = sum(1 for _ in range(sq // n) for _ in range(skv // n) for _ in range(d)) * 2
    _, t = orc.schedule_model(sq, skv, d, n, 1.0, 1.0)
    assert t["compute"] == 2 * madds


# ---------------------------------------------------------------- gradients through the recompute

def _flat_heads(g):
    B, H, S, D = g.shape
    return g.transpose(0, 2, 1, 3).reshape(B * S, H * D)  # column n = h*D + d


def test_recompute_grads_vs_numpy(orc):
    B, S, E, H, D = 2, 5, 12, 3, 4
    y = rnd((B, S, E), 160)
    wk, wv = rnd((H * D, E), 161), rnd((H * D, E), 162)
    gk, gv = rnd((B, H, S, D), 163), rnd((B, H, S, D), 164)
    dW = orc.kv_grad_w(y, gk)
    np.testing.assert_allclose(dW, _flat_heads(gk).T @ y.reshape(B * S, E), rtol=1e-12,
                               atol=1e-13)
    dy = orc.kv_grad_y(gk, gv, wk, wv)
    np.testing.assert_allclose(dy, _flat_heads(gk) @ wk + _flat_heads(gv) @ wv, rtol=1e-12,
                               atol=1e-13)
    np.testing.assert_array_equal(orc.kv_grad_w(y, gk, rows=[7, 0, 11]), dW[[7, 0, 11]])
    np.testing.assert_array_equal(orc.kv_grad_y(gk, gv, wk, wv, rows=[9, 2]), dy[[9, 2]])


def test_recompute_grads_are_adjoints(orc):
    """The gradients are the adjoints of the projection (pinned against numpy
    above and in test_projection_vs_numpy): for any Y and W,
    <g, proj(Y, w)> = <dy(g), Y> and <g, proj(y, W)> = <dW(y, g), W>."""
    B, S, E, H, D = 1, 6, 8, 2, 4
    y, Y = rnd((B, S, E), 170), rnd((B, S, E), 171)
    w, W = rnd((H * D, E), 172), rnd((H * D, E), 173)
    g = rnd((B, H, S, D), 174)
    zero_g, zero_w = np.zeros_like(g), np.zeros_like(w)
    lhs = float(np.sum(g * orc.kv_proj(Y, w, H, D)))
    rhs = float(np.sum(orc.kv_grad_y(g, zero_g, w, zero_w).reshape(B, S, E) * Y))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
    lhs = float(np.sum(g * orc.kv_proj(y, W, H, D)))
    rhs = float(np.sum(orc.kv_grad_w(y, g) * W))
    assert abs(lhs - rhs) <= 1e-12 * max(1.0, abs(lhs))
    # dy is linear in (gk, gv): the V path contributes through wv alone
    dy_k = orc.kv_grad_y(g, zero_g, w, W)
    dy_v = orc.kv_grad_y(zero_g, g, w, W)
    np.testing.assert_allclose(orc.kv_grad_y(g, g, w, W), dy_k + dy_v, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(dy_v, orc.kv_grad_y(g, zero_g, W, w), rtol=0, atol=0)


# ---------------------------------------------------------------- striped causal layout

def stripe_positions(S, n):
    """Sequence position of each row of the striped layout: shard w (rows
    [w*S/n, (w+1)*S/n)) holds positions w, w+n, w+2n, ...  Built by dealing
    the positions 0..S-1 round-robin to the n shards."""
    shards = [[] for _ in range(n)]
    for t in range(S):
        shards[t % n].append(t)
    return np.array([t for sh in shards for t in sh])


def test_striped_causal_is_causal_on_positions(orc):
    """Causal attention over rows in the striped order is ordinary causal
    attention on the sequence, with rows reordered by their positions."""
    for (S, n) in [(12, 3), (16, 4), (10, 1)]:
        B, H, D = 1, 2, 4
        q, k, v = rnd((B, H, S, D), 180), rnd((B, H, S, D), 181), rnd((B, H, S, D), 182)
        pos = stripe_positions(S, n)
        assert sorted(pos.tolist()) == list(range(S))
        inv = np.argsort(pos)  # row of the striped layout holding each position
        O, L = orc.attn_fwd(q, k, v, 0.4, causal=("striped", n))
        # natural order: position t is row inv[t] of the striped tensors
        On, Ln = orc.attn_fwd(q[:, :, inv], k[:, :, inv], v[:, :, inv], 0.4, causal=True)
        np.testing.assert_allclose(O[:, :, inv], On, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(L[:, :, inv], Ln, rtol=1e-13, atol=1e-14)
    # row 0 of the striped layout holds position 0: it sees only itself
    q, k, v = rnd((1, 1, 16, 4), 183), rnd((1, 1, 16, 4), 184), rnd((1, 1, 16, 4), 185)
    O, L = orc.attn_fwd(q, k, v, 0.4, causal=("striped", 4))
    np.testing.assert_allclose(O[:, :, 0], v[:, :, 0], rtol=1e-13)


def test_striped_backward_is_causal_backward_on_positions(orc):
    """The exact gradient over rows in the striped order is the causal
    gradient on the sequence with rows reordered by their positions, and the
    striped gradient of a small case matches torch autograd through an
    explicit position mask."""
    for (S, n) in [(12, 3), (16, 4), (9, 9)]:
        B, H, D = 1, 2, 4
        q, k, v = rnd((B, H, S, D), 190), rnd((B, H, S, D), 191), rnd((B, H, S, D), 192)
        do = rnd((B, H, S, D), 193)
        inv = np.argsort(stripe_positions(S, n))
        r = orc.attn_bwd(q, k, v, do, 0.4, causal=("striped", n))
        rn = orc.attn_bwd(q[:, :, inv], k[:, :, inv], v[:, :, inv], do[:, :, inv], 0.4, causal=True)
        for name in ("dq", "dk", "dv"):
            np.testing.assert_allclose(r[name][:, inv], rn[name], rtol=1e-12, atol=1e-14)
    S, n = 8, 2
    q, k, v = rnd((1, 1, S, 3), 194), rnd((1, 1, S, 3), 195), rnd((1, 1, S, 3), 196)
    do = rnd((1, 1, S, 3), 197)
    pos = stripe_positions(S, n)
    qt, kt, vt = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    s = 0.4 * qt @ kt.transpose(-1, -2)
    s = s.masked_fill(torch.tensor(pos[None, :] > pos[:, None]), float("-inf"))
    (torch.softmax(s, dim=-1) @ vt).backward(torch.tensor(do))
    r = orc.attn_bwd(q, k, v, do, 0.4, causal=("striped", n))
    for name, t in (("dq", qt), ("dk", kt), ("dv", vt)):
        np.testing.assert_allclose(r[name], t.grad.numpy().reshape(1, S, 3), rtol=1e-11, atol=1e-13)
