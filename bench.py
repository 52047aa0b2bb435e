"""Benchmark: ring exact attention forward on one MI355X.

Workload (default): LV-XAttn-shaped cross-attention, batch 1, 32 heads,
S_Q = 2048 text queries against S_KV = 131072 visual keys/values (one GPU's
share), D = 128, bf16 inputs with fp32 accumulation, n = 8 KV shards.
A step is one whole ring forward (every round of the schedule, every block
pair, the merge and the final output) over inputs already resident in HBM.

Prints one JSON line.  `value` is attention TFLOP/s counted as
4 * B * H * S_Q * S_KV * D per step.  `roofline` reports the dominant kernel
against the dense bf16 MFMA peak (2.5 PFLOP/s), its duration measured with
HIP events on the stream the library launches on.  `cpu_baseline` times the
fp64 CPU oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
METRIC = "attention TFLOP/s and % bf16 MFMA peak, S_Q=2K x S_KV=128K d=128, 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_bf16_lvx_2k_128k_traffic.txt")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("fwd.hip", "common.h"):
        with open(os.path.join(ROOT, "ring_exact_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(mode: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source and the same mode; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            a, b = line.split("=", 1)
            kv[a.strip()] = b.strip()
    if kv.get("kernel_hash") != kernel_source_hash() or kv.get("mode") != mode:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(q, k, v, w, rows_per_head: int):
    import numpy as np

    import oracle
    g = np.random.default_rng(w.seed)
    rows = []
    for bh in range(w.B * w.H):
        rows.extend(bh * w.SQ + g.choice(w.SQ, size=rows_per_head, replace=False))
    rows = np.array(sorted(rows), dtype=np.int64)
    qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
    t0 = time.perf_counter()
    oracle.attn_fwd(qc, kc, vc, w.scale, causal=w.causal, rows=rows)
    dt = time.perf_counter() - t0
    flops = 4.0 * w.SKV * w.D * len(rows)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{len(rows)} of {w.B * w.H * w.SQ} query rows ({rows_per_head} per head, "
                      f"all {w.B * w.H} heads) against all {w.SKV} keys, fp64, {dt:.1f} s"}


def _find(d: str, suffix: str) -> str:
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def summarize_traffic(fetch_dir: str, write_dir: str, mode: str, command: str) -> str:
    """Write the committed HBM-traffic summary from two rocprofv3 counter passes
    (FETCH_SIZE, then WRITE_SIZE) of `bench.py --copy-calibration`.  Each counter
    is scaled by what it reads for the 1 GiB copy kernel of the same run."""
    import collections
    import csv

    def read(d, counter):
        per = collections.defaultdict(list)
        for r in csv.DictReader(open(_find(d, "counter_collection.csv"))):
            if r["Counter_Name"] == counter:
                per[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        return per

    fe, wr = read(fetch_dir, "FETCH_SIZE"), read(write_dir, "WRITE_SIZE")
    ck = next(k for k in fe if "copyBuffer" in k)
    kk = next(k for k in fe if "fwd_bf16_kernel" in k)
    gib_kib = (1 << 30) / 1024
    f_factor, w_factor = gib_kib / fe[ck][0], gib_kib / wr[ck][0]
    f_kib = sum(fe[kk][1:]) / len(fe[kk][1:])  # the first launch is a warm-up
    w_kib = sum(wr[kk][1:]) / len(wr[kk][1:])
    fetch_b, write_b = f_kib * 1024 * f_factor, w_kib * 1024 * w_factor
    text = f"""# HBM traffic per launch of {kk} (workload lvx_2k_128k, mode {mode})
# from two rocprofv3 counter passes (FETCH_SIZE, then WRITE_SIZE), KiB per dispatch,
# each scaled by what the same counter reads for a plain 1 GiB copy kernel
# (dst.copy_(src) of 2^29 bf16 elements, run by --copy-calibration in the same process).
# commands (from /tmp, one pass each; then this file is written by
#   python bench.py --mode {mode} --summarize-traffic <fetch_dir> <write_dir>):
#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch_dir> -o run -- {command}
#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write_dir> -o run -- {command}
# raw: FETCH_SIZE {f_kib:.0f} KiB/launch; copy kernel FETCH_SIZE {fe[ck][0]:.0f} KiB for 1048576 KiB moved
#      WRITE_SIZE {w_kib:.0f} KiB/launch; copy kernel WRITE_SIZE {wr[ck][0]:.0f} KiB for 1048576 KiB moved
kernel={kk}
mode={mode}
kernel_hash={kernel_source_hash()}
fetch_factor={f_factor:.4f}
write_factor={w_factor:.4f}
fetch_bytes_per_launch={fetch_b:.0f}
write_bytes_per_launch={write_b:.0f}
hbm_bytes_per_launch={fetch_b + write_b:.0f}
"""
    with open(TRAFFIC_FILE, "w") as f:
        f.write(text)
    return text


def summarize_stats(stats_dir: str, workload: str, command: str, top: int = 8) -> str:
    """Write profiles/kernels_<workload>.txt from a rocprofv3 --kernel-trace --stats run."""
    import csv
    rows = list(csv.DictReader(open(_find(stats_dir, "kernel_stats.csv"))))
    lines = [f"# rocprofv3 kernel statistics, workload {workload}",
             f"# command (from /tmp): rocprofv3 --kernel-trace --stats --output-format csv "
             f"-d <dir> -o run -- {command}",
             "# columns: calls, average us, total ms, percent of GPU time, kernel"]
    for r in rows[:top]:
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:12.1f} "
                     f"{float(r['TotalDurationNs']) / 1e6:10.3f} {float(r['Percentage']):6.2f}  "
                     f"{r['Name'][:160]}")
    text = "\n".join(lines) + "\n"
    with open(os.path.join(ROOT, "profiles", f"kernels_{workload}.txt"), "w") as f:
        f.write(text)
    return text


def summarize_rounds(trace_dirs, labels, workload: str, n: int, command: str) -> str:
    """Write profiles/rounds_<workload>.txt: the duration of each of the last n
    launches of the pair kernel (one per round in ROUNDS mode) from rocprofv3
    --kernel-trace runs, one per label."""
    import csv
    lines = [f"# per-round launches of the pair kernel, workload {workload}, ROUNDS mode, n = {n}",
             f"# command (from /tmp, per layout): rocprofv3 --kernel-trace --output-format csv "
             f"-d <dir> -o run -- {command}",
             "# columns: layout, round 0..n-1 durations in ms, sum"]
    for d, label in zip(trace_dirs, labels):
        rows = list(csv.DictReader(open(_find(d, "kernel_trace.csv"))))
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e6
                for r in rows if "fwd_bf16_kernel" in r["Kernel_Name"]][-n:]
        lines.append(f"{label:12s} " + " ".join(f"{x:6.2f}" for x in durs) + f"   sum {sum(durs):.2f}")
    text = "\n".join(lines) + "\n"
    with open(os.path.join(ROOT, "profiles", f"rounds_{workload}.txt"), "w") as f:
        f.write(text)
    return text


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="lvx_2k_128k")
    ap.add_argument("--mode", default="split", choices=["rounds", "fused", "split", "rounds_transfer"])
    ap.add_argument("--sched", default="kv", choices=["kv", "q"])
    ap.add_argument("--cpu-rows-per-head", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--striped", action="store_true",
                    help="causal workloads: rows in the striped order over the n shards "
                         "(every block pair about half visible)")
    ap.add_argument("--weight-grads", action="store_true",
                    help="recompute workload: also run the gradients through the projection "
                         "(dW_k, dW_v, dy) in every step")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, copy one 1 GiB buffer (a plain copy kernel of "
                         "known size, to calibrate HBM byte counters taken under a profiler)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the profiles/ traffic summary from two rocprofv3 counter passes "
                         "and exit (no GPU use)")
    ap.add_argument("--summarize-stats", metavar="STATS_DIR",
                    help="write profiles/kernels_<workload>.txt from a rocprofv3 --stats run "
                         "and exit (no GPU use)")
    ap.add_argument("--summarize-rounds", nargs=2, metavar=("CONTIGUOUS_DIR", "STRIPED_DIR"),
                    help="write profiles/rounds_<workload>.txt from two rocprofv3 kernel traces "
                         "of ROUNDS mode (causal rows in sequence order, then striped) and exit")
    ap.add_argument("--profiled-command", default="python3 bench.py",
                    help="the command line the summarized profiler runs used")
    args = ap.parse_args()
    if args.summarize_traffic:
        print(summarize_traffic(*args.summarize_traffic, args.mode, args.profiled_command))
        return
    if args.summarize_rounds:
        from ring_exact_attention_amd.inputs import WORKLOADS
        print(summarize_rounds(args.summarize_rounds, ["contiguous", "striped"], args.workload,
                               WORKLOADS[args.workload].n, args.profiled_command))
        return
    if args.summarize_stats:
        name = args.workload + ("_weight_grads" if args.weight_grads else "")
        print(summarize_stats(args.summarize_stats, name, args.profiled_command))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: measures one GPU only (the n ring workers are n KV shards "
              "on one device); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import ring_exact_attention_amd as bwa
    from ring_exact_attention_amd import _bwa
    from ring_exact_attention_amd.inputs import WORKLOADS, make_qkv

    if not os.path.exists(_bwa.LIB_PATH):
        from ring_exact_attention_amd import build as hip_build
        hip_build.build()
    bwa.lib()
    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    recompute = w.E > 0
    if recompute:
        from ring_exact_attention_amd.inputs import make_dout, make_recompute
        y, wk, wv = make_recompute(w, device=dev)
        q, _, _ = make_qkv(w.resized(SKV=1), device=dev)
        do = make_dout(w, device=dev)
        k = torch.empty(w.B, w.H, w.SKV, w.D, dtype=q.dtype, device=dev)
        v = torch.empty_like(k)
        bwa.bwa_kv_recompute(y, wk, wv, w.H, w.D, k=k, v=v)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bmode = "rounds" if args.mode in ("rounds", "rounds_transfer") else "fused"
        bws = torch.empty(max(bwa.ring_bwd_workspace(q, k, w.n, bmode), 1), dtype=torch.uint8,
                          device=dev)
        if args.weight_grads:
            dwk = torch.empty(w.H * w.D, w.E, dtype=torch.float32, device=dev)
            dwv = torch.empty_like(dwk)
            dyf = torch.empty(w.B, w.SKV, w.E, dtype=torch.float32, device=dev)
    else:
        q, k, v = make_qkv(w, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.H, w.SQ, dtype=torch.float32, device=dev)
    nbytes = bwa.ring_fwd_workspace(q, k, w.n, args.mode)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)

    def fwd():
        bwa.bwa_ring_fwd(q, k, v, w.n, args.sched, args.mode,
                         causal=("striped" if args.striped and w.causal else w.causal),
                         scale=w.scale, o=o, lse=lse, workspace=ws)

    def step():
        if recompute:
            # training step of one cross-attention layer with activation recompute:
            # K, V from the shared y, forward, K, V recomputed, backward
            bwa.bwa_kv_recompute(y, wk, wv, w.H, w.D, k=k, v=v)
            fwd()
            bwa.bwa_kv_recompute(y, wk, wv, w.H, w.D, k=k, v=v)
            bwa.bwa_ring_bwd(q, k, v, o, lse, do, w.n, args.sched, bmode, causal=w.causal,
                             scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=bws)
            if args.weight_grads:
                bwa.bwa_kv_recompute_bwd(y, wk, wv, dk, dv, dwk_t=dwk, dwv_t=dwv, dy=dyf)
        else:
            fwd()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step_ms = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    ms = sum(per_step_ms) / len(per_step_ms)

    if w.causal:
        flops = 4.0 * w.B * w.H * w.D * w.SQ * (w.SQ + 1) / 2
    else:
        flops = 4.0 * w.B * w.H * w.SQ * w.SKV * w.D
    if recompute:
        gemm = 2.0 * w.B * w.SKV * w.E * w.H * w.D   # one projection
        flops = flops + 4 * gemm + 2.5 * flops      # fwd + 2x(K, V) recompute + bwd (10 S_Q S_KV D)
        if args.weight_grads:
            flops += 4 * gemm                       # dW_k, dW_v, and dy through both projections
    tflops = flops / (ms * 1e-3) / 1e12
    # compulsory HBM bytes of the forward: read Q, K, V once, write O and LSE
    esz = 2 if w.dtype == "bf16" else 4
    fwd_bytes = (w.B * w.H * (2 * w.SQ + 2 * w.SKV) * w.D * esz + w.B * w.H * w.SQ * 4)

    # Dominant kernel: in fused mode the step is one launch of the block-pair
    # kernel; in rounds mode n launches (one per round) plus a small finalize;
    # in split mode one launch plus the merge.  Per-launch flops are the
    # step's flops divided by the launches of that kernel.
    launches = w.n if args.mode in ("rounds", "rounds_transfer") else 1
    if recompute:
        # several kernels per step (GEMM, forward, backward); report the step as a whole
        roofline = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                    "traffic": None, "kernel": "whole step (gemm_kv, fwd, bwd kernels)",
                    "launches_per_step": None}
        if args.weight_grads:
            roofline["kernel"] = "whole step (gemm_kv, fwd, bwd, gemm_dw, gemm_dy kernels)"
    else:
        # the forward kernel's share of the step: in split mode the merge kernel is
        # the rest; its duration is measured separately below
        fwd_ms = ms
        if args.mode == "split":
            # the step is two launches: every pair's partial, then the ordered
            # merge; time the merge alone on the same workspace and subtract
            from ring_exact_attention_amd._bwa import split_workspace_views
            op, lp = split_workspace_views(ws, w.n, w.B, w.H, w.SQ, w.D)
            em = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            bwa.bwa_merge_partials(op, lp, w.n, args.sched, o=o, lse=lse)
            em[0].record(stream)
            for _ in range(args.steps):
                bwa.bwa_merge_partials(op, lp, w.n, args.sched, o=o, lse=lse)
            em[1].record(stream)
            torch.cuda.synchronize()
            merge = em[0].elapsed_time(em[1]) / args.steps
            fwd_ms = max(ms - merge, 1e-6)
        achieved = (flops / launches) / ((fwd_ms * 1e-3) / launches) / 1e12
        traffic = read_traffic(args.mode) if args.workload == "lvx_2k_128k" else None
        roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                    "traffic": traffic, "kernel": "fwd_bf16_kernel<128>",
                    "launches_per_step": launches,
                    "kernel_ms_per_launch": round(fwd_ms / launches, 4),
                    "other_ms_per_step": round(ms - fwd_ms, 4)}

    out = {
        "metric": METRIC if args.workload == "lvx_2k_128k" else
        f"{'training-step' if recompute else 'attention'} TFLOP/s, {w.name}"
        f"{' with weight gradients' if args.weight_grads else ''}, 1 GPU",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_min": round(min(per_step_ms), 4),
        "ms_per_step_max": round(max(per_step_ms), 4),
        "wall_s_timed": round(wall, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "config": {"workload": w.name, "B": w.B, "H": w.H, "S_Q": w.SQ, "S_KV": w.SKV, "D": w.D,
                   "n_shards": w.n, "schedule": args.sched, "mode": args.mode,
                   "causal": ("striped" if args.striped and w.causal else w.causal),
                   "seed": w.seed},
        "roofline": roofline,
    }
    if not recompute:
        out["hbm_GBps_compulsory"] = round(fwd_bytes / (ms * 1e-3) / 1e9, 1)
        out["hbm_frac_compulsory"] = round(fwd_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
    if args.copy_calibration:
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline and not recompute:
        out["cpu_baseline"] = cpu_baseline(q, k, v, w, args.cpu_rows_per_head)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
