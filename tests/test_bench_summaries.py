"""bench.py's profile summarizers on small synthetic rocprofv3 outputs (CPU).

The stage summary splits a kernel trace and three counter runs of
`bench.py --stage-run` by the marker launches, attributes kernels to stages,
scales the byte counters by what they read for the 1 GiB calibration copy
and derives GB/s and the matrix-core rate; the traffic summary does the same
for the gate GEMM alone.
"""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

GEMM, SEL, SCAT, FLUSH = ("moer::gate_gemm_dma_kernel<128, 256, 2, 2, 4, 3>",
                          "moer::route_rows_kernel<16, true, 1, 2>",
                          "moer::layout_scatter_kernel", "at::native::reduce_kernel")
COPY = "__amd_rocclr_copyBuffer"
US = {GEMM: 60.0, SEL: 12.0, SCAT: 6.0, FLUSH: 9.0}


def _sequence(n_workloads=5):
    seq = [COPY]
    for _ in range(n_workloads):
        for calls in (bench.STAGE_WARMUP, bench.STAGE_CALLS):
            seq.append("moer::" + bench.MARKER)
            for _ in range(calls):
                seq += [FLUSH, GEMM, SEL, SCAT]
    return seq


def _write_trace(d, seq):
    os.makedirs(d)
    t = 0
    with open(os.path.join(d, "run_kernel_trace.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, ["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for name in seq:
            dur = int(US.get(name, 1.0) * 1000)
            w.writerow({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + dur})
            t += dur + 500


def _write_counter(d, seq, counter, value_of):
    os.makedirs(d)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, name in enumerate(seq):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value_of(name)})


def test_stage_summary(tmp_path):
    seq = _sequence()
    _write_trace(str(tmp_path / "t"), seq)
    # FETCH_SIZE reads half the copy's bytes (scale 2), WRITE_SIZE all of them
    _write_counter(str(tmp_path / "f"), seq, "FETCH_SIZE",
                   lambda n: 524288.0 if n == COPY else {GEMM: 1000.0, SEL: 100.0}.get(n, 10.0))
    _write_counter(str(tmp_path / "w"), seq, "WRITE_SIZE",
                   lambda n: 1048576.0 if n == COPY else {GEMM: 50.0}.get(n, 5.0))
    _write_counter(str(tmp_path / "m"), seq, "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                   lambda n: 2.0e6 if n == GEMM else 0.0)
    out = str(tmp_path / "stages.md")
    bench.summarize_stages(str(tmp_path / "t"), str(tmp_path / "f"), str(tmp_path / "w"),
                           str(tmp_path / "m"), out, "cmd")
    rows = [[c.strip() for c in l.strip().strip("|").split("|")]
            for l in open(out).read().splitlines() if l.startswith("| dsv3_group")]
    gemm = next(r for r in rows if r[1] == "gate GEMM")
    assert gemm[2] == "1" and float(gemm[3]) == pytest.approx(60.0)
    read_mb, written_mb = float(gemm[4]), float(gemm[5])
    # the table prints MB with two decimals
    assert read_mb == pytest.approx(1000 * 1024 * 2 / 1e6, abs=0.006)
    assert written_mb == pytest.approx(50 * 1024 / 1e6, abs=0.006)
    gbs = (1000 * 1024 * 2 + 50 * 1024) / 60e-6 / 1e9
    assert float(gemm[6]) == pytest.approx(gbs, abs=1.0)
    tflops = 2.0e6 * 512 / 60e-6 / 1e12
    assert float(gemm[8]) == pytest.approx(tflops, abs=1.0)
    sel = next(r for r in rows if r[1].startswith("selection"))
    assert float(sel[3]) == pytest.approx(12.0) and sel[8] == "—"
    total = next(r for r in rows if "sum of stages" in r[1])
    assert float(total[3].strip("*")) == pytest.approx(78.0)  # the flush is not a stage
    # every workload gets its rows, from its measured calls only
    text = open(out).read()
    for name in bench.STAGE_ORDER:
        assert f"| {name} | gate GEMM | 1 |" in text


def test_split_ignores_warmup_and_unmarked_kernels():
    rows = [("copy", 1), ("k", 2), (bench.MARKER, 0), ("warm", 3), (bench.MARKER, 0),
            ("a", 4), (bench.MARKER, 0), ("warm2", 5), (bench.MARKER, 0), ("b", 6)]
    assert bench._split_stage_rows(rows) == {0: [("a", 4)], 1: [("b", 6)]}


def test_traffic_summary(tmp_path):
    seq = [COPY, GEMM, SEL, GEMM]
    _write_counter(str(tmp_path / "f"), seq, "FETCH_SIZE",
                   lambda n: 524288.0 if n == COPY else 1000.0)
    _write_counter(str(tmp_path / "w"), seq, "WRITE_SIZE",
                   lambda n: 1048576.0 if n == COPY else 100.0)
    out = str(tmp_path / "traffic.json")
    bench.summarize_traffic(str(tmp_path / "f"), str(tmp_path / "w"), out, "cmd")
    res = json.load(open(out))
    assert res["fetch_scale"] == pytest.approx(2.0) and res["write_scale"] == pytest.approx(1.0)
    assert res["bytes_per_launch"] == pytest.approx(1000 * 1024 * 2 + 100 * 1024)
    assert res["gate_gemm_sha256_16"] == bench.gemm_source_hash()


def test_counter_summary(tmp_path):
    # one launch each of the GEMM and the selection kernel per counter run
    seq = [GEMM, SEL]
    vals = {"GRBM_GUI_ACTIVE": {GEMM: 8 * 1000.0, SEL: 8 * 500.0},
            "TCP_TCC_READ_REQ_sum": {GEMM: 4000.0, SEL: 100.0},
            "TCP_TCC_READ_REQ_LATENCY_sum": {GEMM: 4000.0 * 600, SEL: 100.0 * 1200},
            "TCC_HIT_sum": {GEMM: 3.0, SEL: 1.0}, "TCC_MISS_sum": {GEMM: 1.0, SEL: 1.0},
            "TA_TA_BUSY_sum": {GEMM: 256 * 750.0, SEL: 0.0},
            "SQ_INSTS_VALU_MFMA_MOPS_BF16": {GEMM: 1.0e6, SEL: 0.0},
            "SQ_VALU_MFMA_BUSY_CYCLES": {GEMM: 256 * 4 * 1000 * 0.4, SEL: 0.0}}
    dirs = []
    for i, (c, v) in enumerate(vals.items()):
        d = str(tmp_path / f"c{i}")
        _write_counter(d, seq, c, lambda n, v=v: v[n])
        dirs.append(d)
    out = str(tmp_path / "counters.md")
    bench.summarize_counters(dirs, out, "cmd")
    rows = {}
    for l in open(out).read().splitlines():
        cells = [c.strip() for c in l.strip().strip("|").split("|")]
        if len(cells) == 4:
            rows[cells[0]] = cells[1:]
    assert rows["GRBM_GUI_ACTIVE"][0] == "8,000"
    assert rows["cycles per launch (per die)"][:2] == ["1,000", "500"]
    assert rows["L2 read latency, mean (cycles)"][:2] == ["600", "1200"]
    # latency sum / (256 CUs x cycles): 2.4e6 / 256e3 and 1.2e5 / 128e3
    assert rows["L2 reads in flight per CU, mean"][:2] == ["9", "1"]
    assert rows["L2 hit rate"][:2] == ["75.0 %", "50.0 %"]
    assert rows["TA busy (share of CU cycles)"][:2] == ["75 %", "0 %"]
    assert rows["L2 hit rate"][2] == "—"  # no layout kernel in these runs
    # 1e6 x 512 flop in 1000 cycles at 2.4 GHz
    assert rows["bf16 matrix flop per launch"][0] == "5.12e+08"
    assert rows["bf16 matrix rate at 2.4 GHz (TFLOP/s)"][0] == "1229"
    assert rows["matrix cores busy (share of SIMD cycles)"][:2] == ["40 %", "0 %"]


def test_bench_refuses_more_than_one_gpu():
    import subprocess

    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
