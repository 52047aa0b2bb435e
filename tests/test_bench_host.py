"""Host logic of bench.py (no GPU): the one-GPU refusal and the rocprofv3
summarizers that turn profiler output into the files under profiles/, on
small synthetic profiler outputs written here."""
import csv
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture
def profiles(tmp_path, monkeypatch):
    d = tmp_path / "profiles"
    d.mkdir()
    monkeypatch.setattr(bench, "PROFILES", str(d))
    return d


def _bench_log(path, steps, warmup, **extra):
    line = {"metric": bench.METRIC, "value": 1000.0, "unit": "TFLOP/s", "steps": steps,
            "warmup": warmup, "ms_per_step": 4.2, "ms_per_step_min": 4.1, "ms_per_step_max": 4.4,
            "config": {"workload": "lvx_2k_128k", "mode": "split", "S_Q": 2048}}
    line.update(extra)
    path.write_text("some log line\n" + json.dumps(line) + "\n")
    return str(path)


def _trace(dirpath, dispatches):
    """kernel_trace.csv with (dispatch id, kernel, start ns, duration ns) rows."""
    dirpath.mkdir(parents=True, exist_ok=True)
    with open(dirpath / "run_kernel_trace.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for d, k, s, dur in dispatches:
            w.writerow([d, k, s, s + dur])


def _counters(dirpath, rows):
    """counter_collection.csv with (dispatch id, kernel, counter, value) rows."""
    dirpath.mkdir(parents=True, exist_ok=True)
    with open(dirpath / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for r in rows:
            w.writerow(r)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_kernel_stats_leave_out_warmup_dispatches(tmp_path, profiles):
    # 2 warm-up + 3 timed steps; one pair kernel (slow while warming up) and
    # one merge per step
    rows, t, d = [], 0, 0
    for step in range(5):
        for k, dur in (("void bwa::fwd_bf16_kernel<128>(bwa::FwdParams)", 9000 if step < 2 else 3000),
                       ("void bwa::split_merge_kernel<__bf16>(bwa::FwdParams)", 100)):
            rows.append((d, k, t, dur))
            d += 1
            t += dur + 10
    _trace(tmp_path / "trace", rows)
    log = _bench_log(tmp_path / "b.log", steps=3, warmup=2)
    text = bench.summarize_stats(str(tmp_path / "trace"), log, "lvx_2k_128k", "python3 bench.py")
    body = [l.split() for l in text.splitlines() if not l.startswith("#")]
    fwd = next(r for r in body if "fwd_bf16_kernel<128>" in r[-1])
    assert fwd[0] == "1" and float(fwd[1]) == pytest.approx(3.0)  # us, timed steps only
    assert float(fwd[2]) == pytest.approx(3.0) and float(fwd[3]) == pytest.approx(3.0)
    assert "ms_per_step (median) 4.2" in text
    assert (profiles / "kernels_lvx_2k_128k.txt").read_text() == text


def test_counter_summary_reports_l2_hit_rate_and_lds_ratios(tmp_path, profiles):
    rows, cnt, t = [], [], 0
    k = "void bwa::fwd_bf16_kernel<128>(bwa::FwdParams)"
    for d in range(4):  # 1 warm-up + 3 timed steps
        rows.append((d, k, t, 1000))
        t += 2000
        hit = 10.0 if d == 0 else 30.0
        # two instances per counter, as rocprofv3 reports per XCD/SE: summed per dispatch
        for inst in range(2):
            cnt += [(d, k, "TCC_HIT_sum", hit / 2), (d, k, "TCC_MISS_sum", 5.0),
                    (d, k, "SQ_LDS_IDX_ACTIVE", 500.0), (d, k, "SQ_LDS_BANK_CONFLICT", 25.0),
                    (d, k, "SQ_LDS_DATA_FIFO_FULL", 50.0)]
    _trace(tmp_path / "pmc", rows)
    _counters(tmp_path / "pmc", cnt)
    log = _bench_log(tmp_path / "b.log", steps=3, warmup=1)
    text = bench.summarize_pmc(str(tmp_path / "pmc"), log, "lvx_2k_128k", "l2_counters",
                               "python3 bench.py")
    assert "L2 hit rate 0.750" in text  # 30 / (30 + 10): warm-up dispatch left out
    # instances summed per dispatch: 50 / 1000 and 100 / 1000
    assert "LDS bank-conflict cycles / LDS active cycles 0.0500" in text
    assert "LDS data-FIFO-full cycles / LDS active cycles 0.1000" in text
    assert (profiles / "l2_counters_lvx_2k_128k.txt").exists()


def test_mfma_busy_and_clock_from_mfmautil(tmp_path, profiles, monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "h0")
    k = "void bwa::fwd_bf16_kernel<128>(bwa::FwdParams)"
    rows, cnt = [], []
    # duration 4e6 ns; busiest XCD 8e6 cycles (2 GHz); busy cycles 0.5 * 8e6 * 1024
    for d in range(3):
        rows.append((d, k, d * 10 ** 7, 4 * 10 ** 6))
        cnt += [(d, k, "MfmaUtil", 50.0), (d, k, "SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 8e6 * 1024),
                (d, k, "GRBM_GUI_ACTIVE", 8 * 7.9e6), (d, k, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e9)]
    _trace(tmp_path / "pmc", rows)
    _counters(tmp_path / "pmc", cnt)
    log = _bench_log(tmp_path / "b.log", steps=2, warmup=1)
    text = bench.summarize_counters(str(tmp_path / "pmc"), log, "lvx_2k_128k", "python3 bench.py")
    kv = bench._read_kv(str(profiles / "mfma_busy_lvx_2k_128k.txt"))
    assert float(kv["fwd_mfma_busy"]) == pytest.approx(0.5)
    assert float(kv["fwd_clock_ghz"]) == pytest.approx(2.0)
    assert kv["mode"] == "split" and kv["kernel_hash"] == "h0"
    assert bench.read_counters("lvx_2k_128k", "split") == (pytest.approx(0.5), pytest.approx(2.0))
    # a summary taken on other kernel source or in another mode is not used
    assert bench.read_counters("lvx_2k_128k", "fused") == (None, None)
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "h1")
    assert bench.read_counters("lvx_2k_128k", "split") == (None, None)
    assert "0.5120" in text  # executed TFLOP per dispatch: 1e9 MOPS x 512


def test_traffic_scaled_by_the_copy_kernel(tmp_path, profiles, monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "h0")
    copyk, fwdk = "__amd_rocclr_copyBuffer", "void bwa::fwd_bf16_kernel<128>(bwa::FwdParams)"
    gib_kib = (1 << 30) / 1024
    # FETCH_SIZE reads half the bytes a copy moves, WRITE_SIZE all of them
    _counters(tmp_path / "fetch", [(0, fwdk, "FETCH_SIZE", 1.0), (1, fwdk, "FETCH_SIZE", 1000.0),
                                   (2, fwdk, "FETCH_SIZE", 1000.0),
                                   (3, copyk, "FETCH_SIZE", gib_kib / 2)])
    _counters(tmp_path / "write", [(0, fwdk, "WRITE_SIZE", 1.0), (1, fwdk, "WRITE_SIZE", 100.0),
                                   (2, fwdk, "WRITE_SIZE", 100.0), (3, copyk, "WRITE_SIZE", gib_kib)])
    bench.summarize_traffic(str(tmp_path / "fetch"), str(tmp_path / "write"), "shortq_256_256k",
                            "split", "python3 bench.py --copy-calibration")
    kv = bench._read_kv(bench.traffic_file("shortq_256_256k"))
    assert float(kv["fetch_factor"]) == pytest.approx(2.0)
    assert float(kv["write_factor"]) == pytest.approx(1.0)
    assert float(kv["hbm_bytes_per_launch"]) == pytest.approx((1000 * 2 + 100) * 1024)
    assert bench.read_traffic("shortq_256_256k", "split") == pytest.approx(2100 * 1024)
    assert bench.read_traffic("shortq_256_256k", "fused") is None


def test_sq_sweep_ratio(tmp_path, profiles):
    logs = []
    for sq, ms in ((1024, 2.0), (2048, 4.2)):
        logs.append(_bench_log(tmp_path / f"s{sq}.log", steps=5, warmup=1, ms_per_step=ms,
                               value=1.0, config={"S_Q": sq}))
    text = bench.summarize_sweep(logs, "python3 bench.py")
    rows = [l.split() for l in text.splitlines() if not l.startswith("#")]
    assert [r[0] for r in rows] == ["1024", "2048"]
    assert float(rows[1][-1]) == pytest.approx(4.2 / 2.0 / 2)


def test_clamped_counters_give_no_ratio(tmp_path, profiles):
    # LDS active cycles read 2^29 in every dispatch (the counter's limit on a long
    # kernel): the ratios over it are withheld; a natural count is kept
    k = "void bwa::fwd_bf16_kernel<128>(bwa::FwdParams)"
    rows, cnt = [], []
    for d in range(3):  # 1 warm-up + 2 timed steps
        rows.append((d, k, d * 10000, 1000))
        cnt += [(d, k, "SQ_LDS_IDX_ACTIVE", float(1 << 29)), (d, k, "SQ_LDS_BANK_CONFLICT", 0.0),
                (d, k, "SQ_LDS_DATA_FIFO_FULL", 5.0), (d, k, "SQ_INSTS_LDS", 1000.0),
                (d, k, "SQ_WAIT_INST_LDS", 730.0)]
    _trace(tmp_path / "pmc", rows)
    _counters(tmp_path / "pmc", cnt)
    log = _bench_log(tmp_path / "b.log", steps=2, warmup=1)
    text = bench.summarize_pmc(str(tmp_path / "pmc"), log, "lvx_2k_128k", "lds_counters",
                               "python3 bench.py")
    assert "clamped (multiple of 2^24, not a count): SQ_LDS_IDX_ACTIVE" in text
    assert "LDS bank-conflict cycles / LDS active cycles n/a (SQ_LDS_IDX_ACTIVE clamped)" in text
    assert "wave cycles waiting to issue LDS per LDS instruction 0.73" in text
    assert not bench._clamped(123456789.0) and bench._clamped(float(1 << 32))


def test_slot_timer_summary(tmp_path, profiles, monkeypatch):
    import numpy as np
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "h0")
    # 4 workgroups of 256 tiles and one without tiles; group A spends 1000 cycles
    # per tile in its VALU phase and 2000 in its MFMA phase, group B twice that
    rec = np.zeros((5, 2, 6), dtype=np.int64)
    for w in range(4):
        rec[w, 0] = [1000 * 256, 100 * 256, 50 * 256, 2000 * 256, 10 * 256, 256]
        rec[w, 1] = [2000 * 256, 200 * 256, 100 * 256, 4000 * 256, 20 * 256, 256]
    text = bench.summarize_slot_timers(rec, 4.0, 4.2, "lvx_2k_128k", "split",
                                       "python3 bench.py --slot-timers")
    rows = {tuple(l.split()[:2]): [float(x) for x in l.split()[2:]]
            for l in text.splitlines() if not l.startswith("#")}
    assert rows[("A", "valu")] == [1000.0, 1000.0, 1000.0]
    assert rows[("B", "mfma")][0] == 4000.0
    assert rows[("A", "total")][0] == 3160.0 and rows[("B", "total")][0] == 6320.0
    assert "workgroups with tiles 4 (of 5 recorded)" in text
    assert "+5.0%" in text
    assert (profiles / "slot_timers_lvx_2k_128k.txt").read_text() == text
