"""HIP-graph capture of the ring calls (through the C ABI).

The forward with a caller-provided workspace and the allocation-free
backward enqueue only kernels (and, in the transfer mode, device-to-device
copies) on the caller's stream, so a caller can record them once into a
graph and replay it: every launch of the n rounds then costs one graph
launch.  Each test records the call once, then replays it three times with
new inputs written in between (eager work on the same stream) and compares
every replay bitwise with an eager call on the same inputs: the kernels are
deterministic, so a replay that read stale state or skipped a node would
differ.
"""
import pytest
import torch

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


def _fill(gen, *tensors, std=0.5):
    for t in tensors:
        t.copy_((torch.randn(t.shape, generator=gen) * std).to(t.dtype))


def _capture(fn):
    """Warm up on a side stream (as torch's graph capture expects), then record fn."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


@pytest.mark.parametrize("causal", [False, True])
def test_ring_fwd_graph_replays(bwa, causal):
    B, H, SQ, SKV, D, n = (1, 4, 1000, 8192, 128, 8) if not causal else (1, 2, 2048, 2048, 128, 4)
    gen = torch.Generator().manual_seed(21 + causal)
    q = torch.empty(B, H, SQ, D, dtype=torch.bfloat16, device="cuda")
    k = torch.empty(B, H, SKV, D, dtype=torch.bfloat16, device="cuda")
    v = torch.empty_like(k)
    _fill(gen, q, k, v)
    for mode in ("rounds", "fused", "split", "rounds_transfer"):
        for sched in ("kv", "q"):
            log_case(graph="ring_fwd", causal=causal, mode=mode, sched=sched)
            nbytes = bwa.ring_fwd_workspace(q, k, n, mode)
            ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None
            o = torch.empty_like(q)
            lse = torch.empty(B, H, SQ, dtype=torch.float32, device="cuda")
            graph = _capture(lambda: bwa.bwa_ring_fwd(q, k, v, n, sched, mode, causal=causal, o=o,
                                                      lse=lse, workspace=ws))
            for rep in range(3):
                _fill(gen, q, k, v)
                o_ref, lse_ref = bwa.bwa_ring_fwd(q, k, v, n, sched, mode, causal=causal)
                o.zero_()
                graph.replay()
                torch.cuda.synchronize()
                assert torch.equal(o, o_ref), (mode, sched, rep)
                assert torch.equal(lse, lse_ref), (mode, sched, rep)
            del graph


@pytest.mark.parametrize("causal", [False, True])
def test_ring_bwd_noalloc_graph_replays(bwa, causal):
    B, H, SQ, SKV, D, n = (1, 4, 1000, 4096, 128, 4) if not causal else (1, 2, 1024, 1024, 64, 4)
    gen = torch.Generator().manual_seed(31 + causal)
    q = torch.empty(B, H, SQ, D, dtype=torch.bfloat16, device="cuda")
    k = torch.empty(B, H, SKV, D, dtype=torch.bfloat16, device="cuda")
    v, do = torch.empty_like(k), torch.empty_like(q)
    o, lse = torch.empty_like(q), torch.empty(B, H, SQ, dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)

    def inputs():
        _fill(gen, q, k, v)
        _fill(gen, do, std=1.0)
        bwa.bwa_ring_fwd(q, k, v, n, "kv", "fused", causal=causal, o=o, lse=lse)

    inputs()
    for sched in ("kv", "q"):
        log_case(graph="ring_bwd_noalloc", causal=causal, sched=sched)
        graph = _capture(lambda: bwa.bwa_ring_bwd_noalloc(q, k, v, o, lse, do, n, dq, dk, dv,
                                                          sched, "fused", causal=causal))
        for rep in range(3):
            inputs()
            ref = bwa.bwa_ring_bwd(q, k, v, o, lse, do, n, sched, "fused", causal=causal)
            for t in (dq, dk, dv):
                t.zero_()
            graph.replay()
            torch.cuda.synchronize()
            for got, want, name in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
                assert torch.equal(got, want), (name, sched, rep)
        del graph
