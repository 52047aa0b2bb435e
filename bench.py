"""Benchmark: ring exact attention forward on one MI355X.

Workload (default): LV-XAttn-shaped cross-attention, batch 1, 32 heads,
S_Q = 2048 text queries against S_KV = 131072 visual keys/values (one GPU's
share), D = 128, bf16 inputs with fp32 accumulation, n = 8 KV shards.
A step is one whole ring forward (every round of the schedule, every block
pair, the merge and the final output) over inputs already resident in HBM.

Prints one JSON line.  `value` is attention TFLOP/s counted as
4 * B * H * S_Q * S_KV * D per step, from the median step time (min, max and
mean are reported beside it).  `roofline` reports the dominant kernel against
its bound: the dense bf16 MFMA peak (2.5 PFLOP/s) for the compute-bound
workloads, HBM (8 TB/s) for the short-query one, with the kernel's duration
measured with HIP events on the stream the library launches on.  Counter
summaries committed under profiles/ (HBM bytes, MFMA busy fraction, running
clock) are attached when they were taken on the current kernel source.
`cpu_baseline` times the fp64 CPU oracle on a bounded sample of the same
workload.
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
NOMINAL_CLOCK_GHZ = 2.4
SIMDS = 256 * 4  # compute units x SIMDs per CU
METRIC = "attention TFLOP/s and % bf16 MFMA peak, S_Q=2K x S_KV=128K d=128, 1 GPU"
PROFILES = os.path.join(ROOT, "profiles")
# the forward workloads' bound; the rest are compute-bound
HBM_BOUND = {"shortq_256_256k"}
# default ring mode per workload: split everywhere except causal self-attention,
# where split would write n fp32 partials of the whole sequence
DEFAULT_MODE = {"causal_64k": "fused"}


def traffic_file(workload: str) -> str:
    return os.path.join(PROFILES, f"fwd_bf16_{workload}_traffic.txt")


def counters_file(workload: str) -> str:
    return os.path.join(PROFILES, f"mfma_busy_{workload}.txt")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("fwd.hip", "common.h"):
        with open(os.path.join(ROOT, "ring_exact_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _read_kv(path: str) -> dict:
    kv = {}
    if os.path.exists(path):
        for line in open(path):
            if "=" in line and not line.lstrip().startswith("#"):
                a, b = line.split("=", 1)
                kv[a.strip()] = b.strip()
    return kv


def read_traffic(workload: str, mode: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source and the same mode; else None."""
    kv = _read_kv(traffic_file(workload))
    if kv.get("kernel_hash") != kernel_source_hash() or kv.get("mode") != mode:
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_counters(workload: str, mode: str):
    """(MFMA busy fraction, clock GHz) of the forward kernel from the committed
    counter summary, if taken on the current kernel source and mode."""
    kv = _read_kv(counters_file(workload))
    if kv.get("kernel_hash") != kernel_source_hash() or kv.get("mode") != mode:
        return None, None
    try:
        return float(kv["fwd_mfma_busy"]), float(kv["fwd_clock_ghz"])
    except (KeyError, ValueError):
        return None, None


def cpu_baseline(q, k, v, w, rows_per_head: int):
    import numpy as np

    import oracle
    if w.dtype != "bf16":
        # latency-bound fp32 workload: the whole problem, as time per call
        qc, kc, vc = q.cpu(), k.cpu(), v.cpu()
        oracle.attn_fwd(qc, kc, vc, w.scale, causal=w.causal)
        reps = 20
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.attn_fwd(qc, kc, vc, w.scale, causal=w.causal)
        dt = (time.perf_counter() - t0) / reps
        return {"value": round(dt * 1e6, 1), "unit": "us", "cores": oracle.num_threads(),
                "kind": "oracle",
                "sample": f"the whole problem ({w.B * w.H * w.SQ} rows x {w.SKV} keys), fp64, "
                          f"mean of {reps} calls"}
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


def summarize_traffic(fetch_dir: str, write_dir: str, workload: str, mode: str,
                      command: str) -> str:
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
    text = f"""# HBM traffic per launch of {kk} (workload {workload}, mode {mode})
# from two rocprofv3 counter passes (FETCH_SIZE, then WRITE_SIZE), KiB per dispatch,
# each scaled by what the same counter reads for a plain 1 GiB copy kernel
# (dst.copy_(src) of 2^29 bf16 elements, run by --copy-calibration in the same process).
# commands (from /tmp, one pass each; then this file is written by
#   python bench.py --workload {workload} --mode {mode} --summarize-traffic <fetch_dir> <write_dir>):
#   rocprofv3 --pmc FETCH_SIZE --output-format csv -d <fetch_dir> -o run -- {command}
#   rocprofv3 --pmc WRITE_SIZE --output-format csv -d <write_dir> -o run -- {command}
# raw: FETCH_SIZE {f_kib:.0f} KiB/launch; copy kernel FETCH_SIZE {fe[ck][0]:.0f} KiB for 1048576 KiB moved
#      WRITE_SIZE {w_kib:.0f} KiB/launch; copy kernel WRITE_SIZE {wr[ck][0]:.0f} KiB for 1048576 KiB moved
kernel={kk}
workload={workload}
mode={mode}
kernel_hash={kernel_source_hash()}
fetch_factor={f_factor:.4f}
write_factor={w_factor:.4f}
fetch_bytes_per_launch={fetch_b:.0f}
write_bytes_per_launch={write_b:.0f}
hbm_bytes_per_launch={fetch_b + write_b:.0f}
"""
    with open(traffic_file(workload), "w") as f:
        f.write(text)
    return text


def _bench_line(log: str) -> dict:
    """The JSON line bench.py printed into `log`."""
    for line in open(log):
        line = line.strip()
        if line.startswith("{") and '"metric"' in line:
            return json.loads(line)
    raise ValueError(f"no bench JSON line in {log}")


def _short(name: str) -> str:
    name = name.replace("void ", "").replace("bwa::", "")
    return name.split("(")[0][:60]


def _trace_rows(trace_dir: str):
    """(kernel name, duration ns, start ns) of every dispatch, in launch order."""
    import csv
    rows = [(r["Kernel_Name"], int(r["End_Timestamp"]) - int(r["Start_Timestamp"]),
             int(r["Start_Timestamp"]))
            for r in csv.DictReader(open(_find(trace_dir, "kernel_trace.csv")))]
    rows.sort(key=lambda x: x[2])
    return rows


def summarize_stats(trace_dir: str, bench_log: str, name: str, command: str) -> str:
    """Write profiles/kernels_<name>.txt from a rocprofv3 --kernel-trace run of
    bench.py: per kernel, the average over the timed steps only (the first
    `warmup` steps' dispatches of each kernel are left out; they run at lower
    clocks), beside the median step time bench.py measured in that same run."""
    import collections
    b = _bench_line(bench_log)
    steps, warm = b["steps"], b["warmup"]
    per = collections.defaultdict(list)
    for k, dur, _ in _trace_rows(trace_dir):
        per[k].append(dur)
    lines = [f"# rocprofv3 kernel trace, workload {name}; averages over the {steps} timed steps",
             f"# (the first {warm} warm-up steps' dispatches of every kernel are left out)",
             f"# command (from /tmp): rocprofv3 --kernel-trace --output-format csv -d <dir> -o run "
             f"-- {command}",
             f"# the same run's bench.py line: ms_per_step (median) {b['ms_per_step']}, "
             f"min {b.get('ms_per_step_min')}, max {b.get('ms_per_step_max')}, "
             f"value {b['value']} {b['unit']}",
             "# columns: dispatches per step, average us, min us, max us, ms per step, kernel"]
    out = []
    for k, durs in per.items():
        if k.startswith("__amd") or "copyBuffer" in k or "fillBuffer" in k or "elementwise" in k:
            continue
        per_step = len(durs) // (steps + warm) if len(durs) >= steps + warm else 0
        if per_step == 0:
            continue
        timed = durs[warm * per_step:(warm + steps) * per_step]
        avg = sum(timed) / len(timed)
        out.append((avg * per_step, per_step, avg, min(timed), max(timed), k))
    out.sort(reverse=True)
    for tot, per_step, avg, lo, hi, k in out:
        lines.append(f"{per_step:4d} {avg / 1e3:10.1f} {lo / 1e3:10.1f} {hi / 1e3:10.1f} "
                     f"{tot / 1e6:8.3f}  {_short(k)}")
    text = "\n".join(lines) + "\n"
    with open(os.path.join(PROFILES, f"kernels_{name}.txt"), "w") as f:
        f.write(text)
    return text


def summarize_counters(pmc_dir: str, bench_log: str, name: str, command: str) -> str:
    """Write profiles/mfma_busy_<name>.txt from a rocprofv3 --pmc run with
    --kernel-trace: per kernel, over the timed steps' dispatches,
      MFMA busy = MfmaUtil / 100 = SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs),
      clock     = cycles / duration,
    with cycles the GRBM_GUI_ACTIVE of the busiest XCD (recovered from
    MfmaUtil and the summed busy cycles; without MfmaUtil, the XCD-summed
    GRBM_GUI_ACTIVE / 8), and the bf16 MFMA work the kernel executed,
    SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 FLOP."""
    import collections
    import csv
    b = _bench_line(bench_log)
    steps, warm = b["steps"], b["warmup"]
    vals = collections.defaultdict(lambda: collections.defaultdict(float))
    names, starts = {}, {}
    for r in csv.DictReader(open(_find(pmc_dir, "counter_collection.csv"))):
        d = int(r["Dispatch_Id"])
        vals[d][r["Counter_Name"]] += float(r["Counter_Value"])
        names[d] = r["Kernel_Name"]
    durs = {}
    for r in csv.DictReader(open(_find(pmc_dir, "kernel_trace.csv"))):
        d = int(r["Dispatch_Id"])
        durs[d] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        starts[d] = int(r["Start_Timestamp"])
    per = collections.defaultdict(list)
    for d in sorted(vals, key=lambda x: starts.get(x, x)):
        if d in durs:
            per[names[d]].append((durs[d], vals[d]))
    lines = [f"# rocprofv3 counters per kernel, workload {name}; averages over the {steps} timed",
             f"# steps (warm-up dispatches left out).  MFMA busy = rocprofv3's MfmaUtil, i.e.",
             f"# SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs) with cycles the busiest XCD's",
             f"# GRBM_GUI_ACTIVE; clock = cycles / duration; executed TFLOP =",
             f"# SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512.",
             f"# command (from /tmp): rocprofv3 --kernel-trace --pmc MfmaUtil "
             f"SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE SQ_INSTS_VALU_MFMA_MOPS_BF16 "
             f"--output-format csv -d <dir> -o run -- {command}",
             f"# the same run's bench.py line: ms_per_step (median) {b['ms_per_step']}",
             "# columns: dispatches per step, average us, clock GHz, MFMA busy, executed bf16 "
             "TFLOP per dispatch, executed TFLOP/s, kernel"]
    kv = {}
    for k, recs in per.items():
        per_step = len(recs) // (steps + warm) if len(recs) >= steps + warm else 0
        if per_step == 0 or k.startswith("__amd") or "copyBuffer" in k:
            continue
        timed = recs[warm * per_step:(warm + steps) * per_step]
        dur = sum(x[0] for x in timed) / len(timed)
        busy = sum(x[1].get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) for x in timed) / len(timed)
        mops = sum(x[1].get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) for x in timed) / len(timed)
        util = [x[1]["MfmaUtil"] for x in timed if "MfmaUtil" in x[1]]
        if util and busy > 0:
            # MfmaUtil divides by the busiest XCD's GRBM_GUI_ACTIVE: recover those cycles
            frac = sum(util) / len(util) / 100.0
            cyc = busy / (frac * SIMDS) if frac > 0 else 0.0
        else:
            cyc = sum(x[1].get("GRBM_GUI_ACTIVE", 0.0) for x in timed) / len(timed) / 8
            frac = busy / (cyc * SIMDS) if cyc else 0.0
        clock = cyc / dur if dur else 0.0
        tflop = mops * 512 / 1e12
        lines.append(f"{per_step:4d} {dur / 1e3:10.1f} {clock:6.3f} {frac:6.3f} {tflop:8.4f} "
                     f"{tflop / (dur * 1e-9) if dur else 0:9.1f}  {_short(k)}")
        if "fwd_bf16_kernel" in k:
            kv = {"fwd_mfma_busy": f"{frac:.4f}", "fwd_clock_ghz": f"{clock:.4f}",
                  "fwd_avg_us": f"{dur / 1e3:.1f}"}
    if kv:
        lines += [f"kernel_hash={kernel_source_hash()}", f"mode={b['config'].get('mode')}"]
        lines += [f"{a}={v}" for a, v in kv.items()]
    text = "\n".join(lines) + "\n"
    with open(counters_file(name), "w") as f:
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
    with open(os.path.join(PROFILES, f"rounds_{workload}.txt"), "w") as f:
        f.write(text)
    return text


def summarize_pmc(pmc_dir: str, bench_log: str, name: str, tag: str, command: str) -> str:
    """Write profiles/<tag>_<name>.txt: every counter of a rocprofv3 --pmc run
    with --kernel-trace, per kernel, averaged over the timed steps' dispatches
    (values as rocprofv3 reports them per dispatch, summed over its instances)."""
    import collections
    import csv
    b = _bench_line(bench_log)
    steps, warm = b["steps"], b["warmup"]
    vals = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for r in csv.DictReader(open(_find(pmc_dir, "counter_collection.csv"))):
        d = int(r["Dispatch_Id"])
        vals[d][r["Counter_Name"]] += float(r["Counter_Value"])
        names[d] = r["Kernel_Name"]
    starts, durs = {}, {}
    for r in csv.DictReader(open(_find(pmc_dir, "kernel_trace.csv"))):
        d = int(r["Dispatch_Id"])
        starts[d] = int(r["Start_Timestamp"])
        durs[d] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    per = collections.defaultdict(list)
    for d in sorted(vals, key=lambda x: starts.get(x, x)):
        per[names[d]].append((durs.get(d, 0), vals[d]))
    counters = sorted({c for v in vals.values() for c in v})
    lines = [f"# rocprofv3 counters per kernel, workload {name}; averages over the {steps} timed "
             "steps (warm-up dispatches left out)",
             f"# command (from /tmp): rocprofv3 --kernel-trace --pmc {' '.join(counters)} "
             f"--output-format csv -d <dir> -o run -- {command}",
             f"# the same run's bench.py line: ms_per_step (median) {b['ms_per_step']}",
             "# kernel: average us, then counter = value per dispatch"]
    for k, recs in per.items():
        per_step = len(recs) // (steps + warm) if len(recs) >= steps + warm else 0
        if per_step == 0 or k.startswith("__amd") or "copyBuffer" in k or "at::" in k:
            continue
        timed = recs[warm * per_step:(warm + steps) * per_step]
        dur = sum(x[0] for x in timed) / len(timed)
        avg = {c: sum(x[1].get(c, 0.0) for x in timed) / len(timed) for c in counters}
        lines.append(f"{_short(k)}: {dur / 1e3:.1f} us")
        lines.append("    " + "  ".join(f"{c}={v:.4g}" for c, v in avg.items()))
        # a counter that reads a nonzero multiple of 2^24 in any timed dispatch
        # has hit its limit (a natural count is such a multiple one time in 2^24)
        clamped = sorted(c for c in counters if any(_clamped(x[1].get(c, 0.0)) for x in timed))
        if clamped:
            lines.append("    clamped (multiple of 2^24, not a count): " + " ".join(clamped))

        def ratio(label, num, den, fmt):
            if avg.get(den, 0) <= 0 or num not in avg:
                return
            bad = [c for c in (num, den) if c in clamped]
            derived.append(f"{label} n/a ({' '.join(bad)} clamped)" if bad
                           else f"{label} {fmt % (avg[num] / avg[den])}")
        derived = []
        if avg.get("TCC_HIT_sum", 0) + avg.get("TCC_MISS_sum", 0) > 0:
            derived.append("L2 hit rate %.3f"
                           % (avg["TCC_HIT_sum"] / (avg["TCC_HIT_sum"] + avg["TCC_MISS_sum"])))
        ratio("LDS bank-conflict cycles / LDS active cycles", "SQ_LDS_BANK_CONFLICT",
              "SQ_LDS_IDX_ACTIVE", "%.4f")
        ratio("LDS data-FIFO-full cycles / LDS active cycles", "SQ_LDS_DATA_FIFO_FULL",
              "SQ_LDS_IDX_ACTIVE", "%.4f")
        ratio("VALU co-issued during MFMA-busy cycles", "SQ_VALU_MFMA_COEXEC_CYCLES",
              "SQ_VALU_MFMA_BUSY_CYCLES", "%.3f")
        ratio("wave cycles waiting to issue LDS per LDS instruction", "SQ_WAIT_INST_LDS",
              "SQ_INSTS_LDS", "%.2f")
        lines.extend("    " + x for x in derived)
    text = "\n".join(lines) + "\n"
    with open(os.path.join(PROFILES, f"{tag}_{name}.txt"), "w") as f:
        f.write(text)
    return text


def _clamped(v: float) -> bool:
    """A counter value that is a nonzero multiple of 2^24: the counter's limit,
    not a count (some SQ counters stop there on long kernels)."""
    return v > 0 and v == int(v) and int(v) % (1 << 24) == 0


def summarize_sweep(logs, command: str) -> str:
    """Write profiles/sweep_sq_lvx_2k_128k.txt from bench.py lines of the
    headline workload at several S_Q (same S_KV, heads, D, shards)."""
    rows = sorted((_bench_line(f) for f in logs), key=lambda b: b["config"]["S_Q"])
    base = rows[0]
    lines = ["# S_Q sweep at S_KV = 131072, 32 heads, D = 128, n = 8, split mode: the block",
             "# attention's time against the query length at fixed KV length (time grows in",
             "# proportion to S_Q when the path is compute-bound, stays flat when KV streaming",
             "# dominates).",
             f"# command per point: {command} --sq <S_Q>",
             "# columns: S_Q, median ms per step, TFLOP/s, frac of bf16 peak, ms / (ms at the "
             "smallest S_Q) / (S_Q / smallest S_Q)"]
    for b in rows:
        r = (b["ms_per_step"] / base["ms_per_step"]) / (b["config"]["S_Q"] / base["config"]["S_Q"])
        lines.append(f"{b['config']['S_Q']:6d} {b['ms_per_step']:8.3f} {b['value']:8.1f} "
                     f"{b['value'] / PEAK_BF16_TFLOPS:6.3f} {r:6.3f}")
    text = "\n".join(lines) + "\n"
    with open(os.path.join(PROFILES, "sweep_sq_lvx_2k_128k.txt"), "w") as f:
        f.write(text)
    return text


PHASES = ("valu", "staging", "barrier_open", "mfma", "barrier_close")


def summarize_slot_timers(rec, ms_plain: float, ms_timed: float, name: str, mode: str,
                          command: str) -> str:
    """Write profiles/slot_timers_<name>.txt from the forward kernel's phase
    clocks (int64 [workgroups, 2 groups, 6]: five phase sums and the tile
    count, as bwa_fwd_slot_timers returns them) and the step times of the
    default and the diagnostic build."""
    import numpy as np
    rec = np.asarray(rec, dtype=np.float64)
    live = rec[(rec[:, 0, 5] > 0) & (rec[:, 1, 5] > 0)]
    tiles = live[:, 0, 5]
    lines = [f"# forward kernel phase clocks, workload {name}, mode {mode}: shader-clock cycles "
             "(s_memtime)",
             "# per 64-key tile, wave 0 (group A) and wave 4 (group B) of every workgroup, from "
             "the diagnostic",
             "# build (libbwa_slot_timers.so, BWA_SLOT_TIMERS=1) of the same kernel source",
             f"# command: {command}",
             f"# kernel_hash {kernel_source_hash()}",
             f"# workgroups with tiles {len(live)} (of {len(rec)} recorded), tiles per workgroup "
             f"median {np.median(tiles) if len(live) else 0:.0f}",
             f"# step ms (median): default build {ms_plain:.4f}, diagnostic build {ms_timed:.4f} "
             f"({(ms_timed / ms_plain - 1) * 100:+.1f}%: the cost of the clock reads)",
             "# columns: group, phase, cycles per tile: median, 10th and 90th percentile over "
             "workgroups"]
    if not len(live):
        lines.append("no workgroup recorded a tile")
    for g, gname in ((0, "A"), (1, "B")):
        per = live[:, g, :5] / live[:, g, 5:6]
        for i, ph in enumerate(PHASES):
            x = per[:, i]
            lines.append(f"{gname} {ph:14s} {np.median(x):8.0f} {np.percentile(x, 10):8.0f} "
                         f"{np.percentile(x, 90):8.0f}")
        tot = per.sum(axis=1)
        lines.append(f"{gname} {'total':14s} {np.median(tot):8.0f} {np.percentile(tot, 10):8.0f} "
                     f"{np.percentile(tot, 90):8.0f}")
    text = "\n".join(lines) + "\n"
    with open(os.path.join(PROFILES, f"slot_timers_{name}.txt"), "w") as f:
        f.write(text)
    return text


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="lvx_2k_128k")
    ap.add_argument("--mode", default=None,
                    choices=["rounds", "fused", "split", "rounds_transfer"],
                    help="ring mode (default: fused for causal self-attention, else split)")
    ap.add_argument("--sched", default="kv", choices=["kv", "q"])
    ap.add_argument("--sq", type=int, default=None,
                    help="override the workload's query length (S_Q sweep)")
    ap.add_argument("--cpu-rows-per-head", type=int, default=256)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--striped", action="store_true",
                    help="causal workloads: rows in the striped order over the n shards "
                         "(every block pair about half visible)")
    ap.add_argument("--weight-grads", action="store_true",
                    help="recompute workload: also run the gradients through the projection "
                         "(dW_k, dW_v, dy) in every step")
    ap.add_argument("--graph", action="store_true",
                    help="record one step into a HIP graph (torch.cuda.CUDAGraph over the "
                         "library's stream) and time its replays instead of eager calls")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed steps, copy one 1 GiB buffer (a plain copy kernel of "
                         "known size, to calibrate HBM byte counters taken under a profiler)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the profiles/ traffic summary from two rocprofv3 counter passes "
                         "and exit (no GPU use)")
    ap.add_argument("--summarize-stats", nargs=2, metavar=("TRACE_DIR", "BENCH_LOG"),
                    help="write profiles/kernels_<workload>.txt from a rocprofv3 --kernel-trace "
                         "run and the bench line it printed, and exit (no GPU use)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("PMC_DIR", "BENCH_LOG"),
                    help="write profiles/mfma_busy_<workload>.txt from a rocprofv3 --pmc "
                         "--kernel-trace run and the bench line it printed, and exit")
    ap.add_argument("--summarize-pmc", nargs=3, metavar=("PMC_DIR", "BENCH_LOG", "TAG"),
                    help="write profiles/<TAG>_<workload>.txt with every counter of a rocprofv3 "
                         "--pmc --kernel-trace run, per kernel, and exit")
    ap.add_argument("--summarize-sweep", nargs="+", metavar="BENCH_LOG",
                    help="write profiles/sweep_sq_lvx_2k_128k.txt from bench lines at several "
                         "S_Q and exit")
    ap.add_argument("--summarize-rounds", nargs=2, metavar=("CONTIGUOUS_DIR", "STRIPED_DIR"),
                    help="write profiles/rounds_<workload>.txt from two rocprofv3 kernel traces "
                         "of ROUNDS mode (causal rows in sequence order, then striped) and exit")
    ap.add_argument("--slot-timers", action="store_true",
                    help="forward workloads: time the steps with the default library and with "
                         "its diagnostic build (phase clocks in the forward kernel), then write "
                         "profiles/slot_timers_<workload>.txt from the clocks of the last step "
                         "and exit")
    ap.add_argument("--profiled-command", default="python3 bench.py",
                    help="the command line the summarized profiler runs used")
    args = ap.parse_args()
    mode = args.mode or DEFAULT_MODE.get(args.workload, "split")
    name = args.workload + ("_weight_grads" if args.weight_grads else "") + \
        ("_striped" if args.striped else "")
    if args.summarize_traffic:
        print(summarize_traffic(*args.summarize_traffic, args.workload, mode,
                                args.profiled_command))
        return
    if args.summarize_rounds:
        from ring_exact_attention_amd.inputs import WORKLOADS
        print(summarize_rounds(args.summarize_rounds, ["contiguous", "striped"], args.workload,
                               WORKLOADS[args.workload].n, args.profiled_command))
        return
    if args.summarize_stats:
        print(summarize_stats(*args.summarize_stats, name, args.profiled_command))
        return
    if args.summarize_counters:
        print(summarize_counters(*args.summarize_counters, name, args.profiled_command))
        return
    if args.summarize_pmc:
        d, log, tag = args.summarize_pmc
        print(summarize_pmc(d, log, name, tag, args.profiled_command))
        return
    if args.summarize_sweep:
        print(summarize_sweep(args.summarize_sweep, args.profiled_command))
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
    if args.sq:
        w = w.resized(SQ=args.sq, SKV=w.SKV if not w.causal else args.sq)
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
        bmode = "rounds" if mode in ("rounds", "rounds_transfer") else "fused"
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
    nbytes = bwa.ring_fwd_workspace(q, k, w.n, mode)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    causal = "striped" if args.striped and w.causal else w.causal

    def fwd():
        bwa.bwa_ring_fwd(q, k, v, w.n, args.sched, mode, causal=causal, scale=w.scale, o=o,
                         lse=lse, workspace=ws)

    def step():
        if recompute:
            # training step of one cross-attention layer with activation recompute:
            # K, V from the shared y, forward, K, V recomputed, backward
            bwa.bwa_kv_recompute(y, wk, wv, w.H, w.D, k=k, v=v)
            fwd()
            bwa.bwa_kv_recompute(y, wk, wv, w.H, w.D, k=k, v=v)
            bwa.bwa_ring_bwd(q, k, v, o, lse, do, w.n, args.sched, bmode, causal=causal,
                             scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=bws)
            if args.weight_grads:
                bwa.bwa_kv_recompute_bwd(y, wk, wv, dk, dv, dwk_t=dwk, dwv_t=dwv, dy=dyf)
        else:
            fwd()

    stream = torch.cuda.current_stream(dev)
    if args.slot_timers:
        if recompute or w.dtype != "bf16":
            print("bench.py: --slot-timers covers the bf16 forward workloads", file=sys.stderr)
            sys.exit(2)

        def median_ms():
            for _ in range(args.warmup):
                step()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
            ev[0].record(stream)
            for i in range(args.steps):
                step()
                ev[i + 1].record(stream)
            torch.cuda.synchronize()
            xs = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
            return xs[len(xs) // 2]

        default_lib = _bwa.LIB_PATH
        ms_plain = median_ms()
        _bwa.use_library(_bwa.SLOT_TIMERS_LIB_PATH)
        ms_timed = median_ms()
        rec = _bwa.fwd_slot_timers()
        _bwa.use_library(default_lib)
        command = "python3 bench.py " + " ".join(sys.argv[1:])
        print(summarize_slot_timers(rec, ms_plain, ms_timed, name, mode, command), flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.graph:
        # every buffer of a step is allocated above, so a step records as kernels
        # (and, in the transfer mode, device copies) only
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        step = graph.replay  # noqa: F811  (the timed loop below replays the graph)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step_ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps))
    mid = len(per_step_ms) // 2
    ms = (per_step_ms[mid] if len(per_step_ms) % 2 else
          0.5 * (per_step_ms[mid - 1] + per_step_ms[mid]))
    ms_mean = sum(per_step_ms) / len(per_step_ms)

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
    # in split mode one launch plus the merge.  Per-launch work is the step's
    # work divided by the launches of that kernel.
    launches = w.n if mode in ("rounds", "rounds_transfer") else 1
    if w.dtype != "bf16":
        # fp32 tiny workload: launch- and latency-bound (a few microseconds of work),
        # reported as time per call; no roofline claim
        roofline = {"bound": "latency", "achieved": None, "peak": None, "unit": "us",
                    "frac": None, "traffic": None, "kernel": f"fwd_f32_kernel<{w.D}>",
                    "launches_per_step": w.n if mode in ("rounds", "rounds_transfer") else 1,
                    "us_per_step": round(ms * 1e3, 2)}
    elif recompute:
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
        part_bytes = 0
        if mode == "split":
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
            part_bytes = w.n * w.B * w.H * w.SQ * (w.D + 1) * 4  # partials written
        kernel_ms = fwd_ms / launches
        traffic = read_traffic(args.workload, mode) if not args.sq else None
        busy, clock = read_counters(args.workload, mode) if not args.sq else (None, None)
        if args.workload in HBM_BOUND:
            # algorithmic bytes of one pair-kernel launch: Q, K, V read once, the
            # partials (split) or the output and LSE written
            alg = (w.B * w.H * (w.SQ + 2 * w.SKV) * w.D * esz +
                   (part_bytes if part_bytes else w.B * w.H * w.SQ * (w.D * esz + 4)))
            achieved = alg / launches / (kernel_ms * 1e-3) / 1e9
            roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                        "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                        "traffic": traffic, "algorithmic_bytes_per_launch": alg // launches,
                        "mfma_frac": round(flops / (fwd_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        else:
            achieved = (flops / launches) / (kernel_ms * 1e-3) / 1e12
            roofline = {"bound": "mfma", "achieved": round(achieved, 2),
                        "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic}
        cm = 2 if causal == "striped" else (1 if causal else 0)  # the kernel's causal instance
        roofline.update({"kernel": f"fwd_bf16_kernel<{w.D}, {cm}>", "launches_per_step": launches,
                         "kernel_ms_per_launch": round(kernel_ms, 4),
                         "other_ms_per_step": round(ms - fwd_ms, 4),
                         "mfma_busy_profiled": busy, "clock_ghz_profiled": clock})

    latency = w.dtype != "bf16"
    out = {
        "metric": METRIC if (args.workload == "lvx_2k_128k" and not args.sq) else
        (f"attention time per call (us), {w.name}, 1 GPU" if latency else
         f"{'training-step' if recompute else 'attention'} TFLOP/s, {w.name}"
         f"{' with weight gradients' if args.weight_grads else ''}"
         f"{f' at S_Q={w.SQ}' if args.sq else ''}, 1 GPU"),
        "value": round(ms * 1e3, 2) if latency else round(tflops, 2),
        "unit": "us" if latency else "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_min": round(per_step_ms[0], 4),
        "ms_per_step_max": round(per_step_ms[-1], 4),
        "ms_per_step_mean": round(ms_mean, 4),
        "wall_s_timed": round(wall, 4),
        "higher_is_better": not latency,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "frac_of_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "config": {"workload": w.name, "B": w.B, "H": w.H, "S_Q": w.SQ, "S_KV": w.SKV, "D": w.D,
                   "n_shards": w.n, "schedule": args.sched, "mode": mode, "causal": causal,
                   "seed": w.seed, "graph": args.graph},
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
    if not args.no_cpu_baseline and not recompute and not args.sq:
        out["cpu_baseline"] = cpu_baseline(q, k, v, w, args.cpu_rows_per_head)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
