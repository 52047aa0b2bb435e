"""The allocation-free backward (bwa_ring_bwd_noalloc) against bwa_ring_bwd.

Through the C ABI: two calls in a row on one GPU, the second with a smaller
input, each compared with the workspace entry point (bitwise: the kernels are
shared and the static scratch array only replaces the workspace) and with the
oracle under the element-wise gradient bounds.  The first call of the process
looks the array's device address up.
"""
import math

import pytest
import torch

from tests.parity import check_grad, dq_row_allowance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def bwa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_exact_attention_amd as m
    m.lib()
    return m


def _case(B, H, SQ, SKV, D, seed):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(B, H, SQ, D, generator=g) * 0.5).bfloat16()
    k = (torch.randn(B, H, SKV, D, generator=g) * 0.5).bfloat16()
    v = (torch.randn(B, H, SKV, D, generator=g) * 0.5).bfloat16()
    do = torch.randn(B, H, SQ, D, generator=g).bfloat16()
    return q, k, v, do


@pytest.mark.parametrize("causal", [False, True])
def test_noalloc_matches_workspace_entry_point(bwa, orc, causal):
    shapes = [(2, 3, 640, 640 if causal else 2000, 128, 4, 11),  # first call
              (1, 2, 300, 300 if causal else 700, 128, 3, 12)]   # smaller, same array
    for (B, H, SQ, SKV, D, n, seed) in shapes:
        print(f"case: noalloc B={B} H={H} SQ={SQ} SKV={SKV} D={D} n={n} causal={causal}",
              flush=True)
        scale = 1 / math.sqrt(D)
        q, k, v, do = _case(B, H, SQ, SKV, D, seed)
        qd, kd, vd, dod = q.cuda(), k.cuda(), v.cuda(), do.cuda()
        o, lse = bwa.bwa_ring_fwd(qd, kd, vd, n, "kv", "fused", causal=causal, scale=scale)
        ref = bwa.bwa_ring_bwd(qd, kd, vd, o, lse, dod, n, "kv", "fused", causal=causal,
                               scale=scale)
        outs = (torch.full_like(qd, float("nan")), torch.full_like(kd, float("nan")),
                torch.full_like(vd, float("nan")))
        got = bwa.bwa_ring_bwd_noalloc(qd, kd, vd, o, lse, dod, n, *outs, sched="kv",
                                       mode="fused", causal=causal, scale=scale)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b)
        exact = orc.attn_bwd(q, k, v, do, scale, causal)
        extra = dq_row_allowance(orc, q, k, v, do, scale, causal)
        for name, x in zip(("dq", "dk", "dv"), got):
            check_grad(x.reshape(exact[name].shape), exact[name], f"noalloc {name} {SQ}x{SKV}",
                       row_extra=extra if name == "dq" else None)


def test_noalloc_rejects_rounds(bwa):
    q, k, v, do = (x.cuda() for x in _case(1, 1, 64, 64, 128, 3))
    o, lse = bwa.bwa_ring_fwd(q, k, v, 2)
    outs = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    with pytest.raises(bwa.BwaError, match="ROUNDS"):
        bwa.bwa_ring_bwd_noalloc(q, k, v, o, lse, do, 2, *outs, mode="rounds")
