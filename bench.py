"""Router hot-path benchmark on one MI355X.

One step = one pass of the whole hot path over one batch of the
DeepSeek-V3-style router (16384 tokens, d=7168, 256 experts in 8 groups of
32, keep 4 groups, top-8, sigmoid, selection bias):
  moer_route (gate GEMM, scores, group-limited top-k, weights, per-token and
  batch-mean entropy, counts/offsets/perm/inv_perm, and, fused into the same
  call, the load statistics and the in-place sign-step bias update).
Inputs are resident in HBM before timing; x rotates over three distinct
batches (705 MB in all, larger than the 256 MB last-level cache) so each
step streams its batch from HBM. After the W warm-up steps, untimed steps
continue for CLOCK_RAMP_S of wall time so the timed region starts at the
chip's steady clocks.

Prints ONE JSON line with the throughput (routed tokens/s, from K
uninstrumented steps), the roofline of the dominant kernel (the gate GEMM:
HIP events around its launch on the route's stream, over a second pass of K
steps, since the events themselves cost a few us per step; less the time an
empty event pair reads on the same stream) and the CPU oracle timed on the
host cores.
"""
import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
# the gate GEMM kernel's sources: a change to any of them voids the counters
GEMM_SRCS = [os.path.join(ROOT, "top_expert_routing_gate_amd", "csrc", f)
             for f in ("gate_gemm.hip", "gemm_pipeline.hpp", "moer_internal.hpp")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "route_dsv3_traffic.json")
METRIC = "routed tokens/s, 16k tok × 256 experts top-8; % of MFMA/HBM roofline"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="dsv3_group")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--overlap", action="store_true",
                   help="alternate two streams so step i+1's gate GEMM overlaps step i's "
                        "selection and layout (measured slower: the GEMM needs every CU)")
    p.add_argument("--no-dispatch-combine", action="store_true",
                   help="skip timing the local dispatch and weighted combine that follow the "
                        "route (reported beside the route, not part of its step)")
    p.add_argument("--route-only", action="store_true",
                   help="time the route step only (no dispatch/combine, forcible-layout, "
                        "capacity or balance-step timings): for counter profiles of the step")
    p.add_argument("--no-forcible", action="store_true",
                   help="skip timing the layout on forcibly balanced ids against the routed ids")
    p.add_argument("--report", metavar="OUT_MD",
                   help="per-workload report (all five router shapes): medians and p10/p90 with "
                        "the last-level cache flushed between calls, roofline shares, HIP-graph "
                        "replay for the small batches, the collapse workload's 100-iteration "
                        "balancing series, and the oracle at all cores and at one core")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run one plain 1 GiB device copy (counter calibration)")
    p.add_argument("--summarize-trace", metavar="DIR",
                   help="write a per-kernel table from a rocprofv3 --kernel-trace --stats dir")
    p.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="calibrated HBM bytes per gate-GEMM launch from two --pmc runs")
    p.add_argument("--stage-run", action="store_true",
                   help="route every workload shape STAGE_CALLS times (last-level cache flushed "
                        "between calls), with a marker launch before each workload's warm-up "
                        "and before its measured calls, for per-stage rocprofv3 runs")
    p.add_argument("--summarize-stages", nargs=4,
                   metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "MFMA_DIR"),
                   help="per-workload, per-stage table (us, HBM bytes and GB/s, MFMA rate) from "
                        "a --kernel-trace run and three --pmc runs of --stage-run")
    p.add_argument("--summarize-counters", nargs="+", metavar="PMC_DIR",
                   help="per-launch averages of every counter in these --pmc runs for the "
                        "gate GEMM, selection and layout kernels, with the memory-path "
                        "figures derived from them")
    p.add_argument("--command", default="", help="profiling command recorded in a summary")
    p.add_argument("--out", help="output file of a summary")
    return p.parse_args()


COPY_BYTES = 1 << 30
# After idling, the chip needs ~10-20 ms of load to reach its steady clocks
# (measured on the 16k-token batch: the first 100 back-to-back steps average
# 97 us, then 86-87 us); untimed calls fill this much wall time before any
# timed region.
CLOCK_RAMP_S = 0.06


def clock_ramp(torch, fn, seconds=CLOCK_RAMP_S, batch=20):
    """Untimed calls of fn() until `seconds` of wall time have passed; returns
    how many were made."""
    t0, n = time.perf_counter(), 0
    while True:
        for _ in range(batch):
            fn()
            n += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= seconds:
            return n


def summarize_trace(d, out, command, steps=None, warmup=None):
    """Per-kernel table from a rocprofv3 --kernel-trace --stats directory; with
    the profiled run's steps and warmup, also the gate GEMM over the
    event-timed pass (its last `steps` launches of the route), the figure the
    bench line's roofline uses."""
    import csv
    import glob
    import statistics

    stats = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    rows = list(csv.DictReader(open(stats[0])))
    lines = ["# Kernel trace: bench.py on the DeepSeek-V3-style 16k-token batch", "",
             "Route steps (gate GEMM, selection, layout; warmup, value pass and event-timed "
             "pass), then the variants the bench line reports beside the route (dispatch and "
             "combine, layout on routed and balanced ids, capacity-limited routing, balancing "
             "step).", "",
             "Command (from /tmp, TMPDIR=/tmp):", "", "```", command, "```", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "").replace("|", "/")
        name = name.split("(")[0] if "moer::" in name else name
        lines.append(f"| `{name[:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f} |")
    traces = glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True)
    if traces and steps:
        tr = sorted(csv.DictReader(open(traces[0])), key=lambda r: int(r["Start_Timestamp"]))
        g = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
             for r in tr if "gate_gemm" in r["Kernel_Name"]]
        # launches: warmup, value pass, event-timed pass, then the variants'
        ev = g[warmup + steps:warmup + 2 * steps]
        lines += ["", f"Gate GEMM launches in order: {len(g)}; the event-timed pass "
                      f"(launches {warmup + steps}..{warmup + 2 * steps - 1}): average "
                      f"{statistics.mean(ev):.2f} us, median {statistics.median(ev):.2f} us; "
                      f"value pass: average {statistics.mean(g[warmup:warmup + steps]):.2f} us."]
        # the route steps launch each of their kernels once per step, before
        # any variant runs: the value pass is launches [warmup, warmup + steps)
        # of each
        step_rows = ["", "Per route step, value pass (launches "
                         f"{warmup}..{warmup + steps - 1} of each kernel; the table above "
                         "also averages the variants' launches):", "",
                     "| kernel | avg us | median us |", "|---|---|---|"]
        for key in ("gate_gemm", "route_rows", "route_small", "layout_scatter"):
            k = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
                 for r in tr if key in r["Kernel_Name"]][warmup:warmup + steps]
            if k:
                step_rows.append(f"| {key} | {statistics.mean(k):.2f} | "
                                 f"{statistics.median(k):.2f} |")
        # gaps: first kernel start to last kernel end of each value-pass step
        starts = [int(r["Start_Timestamp"]) for r in tr if "gate_gemm" in r["Kernel_Name"]]
        ends = [int(r["End_Timestamp"]) for r in tr if "layout_scatter" in r["Kernel_Name"]]
        if len(starts) >= warmup + steps and len(ends) >= warmup + steps:
            span = [(ends[i] - starts[i]) / 1e3 for i in range(warmup, warmup + steps)]
            step_rows += ["", f"Gate GEMM start to layout end, per value-pass step: average "
                              f"{statistics.mean(span):.2f} us, median "
                              f"{statistics.median(span):.2f} us."]
        lines += step_rows
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


def _counter_rows(d, counter):
    import csv
    import glob

    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    out = []
    for fn in files:
        for r in csv.DictReader(open(fn)):
            if r["Counter_Name"] == counter:
                out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


MFMA_BF16_PEAK = 2.517e15  # MI355X dense bf16 matrix peak, flop/s
STAGE_ORDER = ["tiny_softmax", "mixtral_top2", "dsv3_group", "collapse_balance", "decode_layers"]
STAGE_WARMUP, STAGE_CALLS = 5, 20
MARKER = "balanced_indices_kernel"  # the stage run's marker launch
STAGES = [("gate_gemm", "gate GEMM"),
          ("route_small", "gate GEMM + selection (one launch, at most 16 experts)"),
          ("route_layer", "the whole call in one workgroup per layer (GEMM, selection, layout, "
                          "statistics, bias update)"),
          ("route_rows", "selection (scores, top-k, weights, entropy, histogram)"),
          ("score_topk", "selection (scores, top-k, weights, entropy, histogram)"),
          ("layout_count", "histogram of supplied ids"),
          ("layout_scatter", "scan + scatter (+ batch entropy, statistics, bias update)"),
          ("zero_ints", "clear counters")]


def _stage_of(kernel):
    for key, label in STAGES:
        if key in kernel:
            return label
    return None


def _split_stage_rows(rows):
    """rows: (kernel name, value) in dispatch order. Returns {workload index:
    [(name, value)]} for the measured calls: the run launches a marker before
    each workload's warm-up and another before its measured calls."""
    per, marks = {}, 0
    for name, v in rows:
        if MARKER in name:
            marks += 1
            continue
        if marks > 0 and marks % 2 == 0:
            per.setdefault(marks // 2 - 1, []).append((name, v))
    return per


def run_stage_calls(args):
    """The route call of every workload shape (the bench step: route, fused
    load statistics and bias update), STAGE_CALLS measured calls each after
    STAGE_WARMUP warm-up calls, with a 512 MB read between calls so the
    last-level cache holds none of the inputs; a 1 GiB copy first calibrates
    the byte counters."""
    import torch

    import top_expert_routing_gate_amd as moer
    import workloads

    dev = torch.device("cuda:0")
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    bcopy = torch.empty_like(a)
    bcopy.copy_(a)
    torch.cuda.synchronize()
    del a, bcopy
    flush = torch.ones(256 << 20, dtype=torch.float16, device=dev)
    for name in STAGE_ORDER:
        wl = workloads.WORKLOADS[name]
        print(f"[stages] {name}", file=sys.stderr, flush=True)
        W, b0, off, gen = workloads.make_router(wl)
        x = workloads.make_hidden(wl, gen=gen)
        L, T, Kt, Nb = wl.n_layers, wl.T, wl.Kt, wl.Nb
        desc = moer.make_desc(n_layers=L, T=T, d=wl.d, N=wl.N, K=wl.K, n_groups=wl.n_groups,
                              topk_groups=wl.topk_groups, n_shared=wl.n_shared,
                              score_fn=wl.score_fn, dtype=wl.dtype)
        i32, f32 = dict(dtype=torch.int32, device=dev), dict(dtype=torch.float32, device=dev)
        bias = b0.clone().to(dev)
        outs = dict(topk_idx=torch.empty(L, T, Kt, **i32), topk_w=torch.empty(L, T, Kt, **f32),
                    tok_entropy=torch.empty(L, T, **f32), agg_entropy=torch.empty(L, **f32),
                    counts=torch.empty(L, Nb, **i32), offsets=torch.empty(L, Nb + 1, **i32),
                    perm=torch.empty(L, T * Kt, **i32), inv_perm=torch.empty(L, T * Kt, **i32))
        ws = torch.empty(max(1, moer.moer_route_workspace_bytes(desc)), dtype=torch.uint8,
                         device=dev)
        call = moer.PreparedRoute(desc, workspace=ws, x=x.to(dev), w_gate=W.to(dev), bias=bias,
                                  logit_offset=None if off is None else off.to(dev),
                                  load_stats=torch.empty(L, 64, dtype=torch.uint8, device=dev),
                                  bias_update=bias, bias_update_u=1e-3, **outs)
        for calls in (STAGE_WARMUP, STAGE_CALLS):
            moer.balanced_indices(1, 1, 1, device=dev)  # marker
            if calls == STAGE_WARMUP:
                clock_ramp(torch, call)  # between the markers: not measured
            for _ in range(calls):
                flush.max()
                call()
        torch.cuda.synchronize()
    print("[stages] done", file=sys.stderr, flush=True)


def summarize_stages(trace_dir, fetch_dir, write_dir, mfma_dir, out, command):
    import csv
    import glob
    import statistics

    traces = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    tr = sorted(csv.DictReader(open(traces[0])), key=lambda r: int(r["Start_Timestamp"]))
    dur = _split_stage_rows([(r["Kernel_Name"],
                              (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
                             for r in tr])

    def counter(d, name):
        rows = []
        for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            rows += [r for r in csv.DictReader(open(fn)) if r["Counter_Name"] == name]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        copy = [float(r["Counter_Value"]) for r in rows if "copyBuffer" in r["Kernel_Name"]]
        return _split_stage_rows([(r["Kernel_Name"], float(r["Counter_Value"])) for r in rows]), copy

    fetch, fcopy = counter(fetch_dir, "FETCH_SIZE")
    write, wcopy = counter(write_dir, "WRITE_SIZE")
    mops, _ = counter(mfma_dir, "SQ_INSTS_VALU_MFMA_MOPS_BF16")
    # counters read KiB; scale each by what it reads for the known 1 GiB copy
    fscale = COPY_BYTES / (max(fcopy) * 1024.0)
    wscale = COPY_BYTES / (max(wcopy) * 1024.0)

    def by_stage(rows):
        acc = {}
        for name, v in rows:
            st = _stage_of(name)
            if st is not None:
                acc.setdefault(st, []).append(v)
        return acc

    lines = ["# Route stages on every workload shape: time, HBM bytes, matrix-core rate", "",
             "Commands (from /tmp, TMPDIR=/tmp; R = repository root): one kernel-trace run and "
             "three counter runs of the same program:", "", "```", command, "```", "",
             f"Each workload: {STAGE_WARMUP} warm-up calls, then {STAGE_CALLS} measured calls of "
             "the bench step (route + fused load statistics + bias update), with a 512 MB read "
             "between calls so the last-level cache holds none of the inputs. Time per launch "
             "comes from the kernel trace. Bytes per launch are FETCH_SIZE + WRITE_SIZE (HBM "
             f"side of the L2). Each is scaled by what it reads for a plain 1 GiB copy "
             f"(fetch x{fscale:.3f}, write x{wscale:.3f}). GB/s = bytes / time; peaks 8 TB/s HBM, "
             "2.517 PFLOP/s dense bf16 (MFMA flop = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512).", "",
             "| workload | stage | launches / call | us / launch | read MB | written MB | GB/s | "
             "% of 8 TB/s | MFMA TFLOP/s | % of bf16 peak |",
             "|---|---|---|---|---|---|---|---|---|---|"]
    for i, name in enumerate(STAGE_ORDER):
        if i not in dur:
            continue
        d_st, f_st = by_stage(dur[i]), by_stage(fetch.get(i, []))
        w_st, m_st = by_stage(write.get(i, [])), by_stage(mops.get(i, []))
        total = 0.0
        for _, label in STAGES:
            if label not in d_st:  # absent, or already reported (two kernels share a label)
                continue
            us = statistics.mean(d_st[label])
            n = len(d_st[label]) / STAGE_CALLS
            total += us * n
            rb = statistics.mean(f_st[label]) * 1024.0 * fscale if label in f_st else float("nan")
            wb = statistics.mean(w_st[label]) * 1024.0 * wscale if label in w_st else float("nan")
            gbs = (rb + wb) / (us * 1e-6) / 1e9
            mf = ""
            if label in m_st and statistics.mean(m_st[label]) > 0:
                tf = statistics.mean(m_st[label]) * 512 / (us * 1e-6)
                mf = f"{tf / 1e12:.0f} | {100 * tf / MFMA_BF16_PEAK:.0f} %"
            else:
                mf = "— | —"
            lines.append(f"| {name} | {label} | {n:g} | {us:.2f} | {rb / 1e6:.2f} | "
                         f"{wb / 1e6:.2f} | {gbs:.0f} | {100 * gbs / HBM_PEAK_GBS:.1f} % | {mf} |")
            d_st.pop(label)
        lines.append(f"| {name} | **sum of stages** | | **{total:.1f}** | | | | | | |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


N_CU, N_XCD = 256, 8  # MI355X compute units and accelerator dies
COUNTER_KERNELS = [("gate_gemm", "gate GEMM"), ("route_rows", "selection"),
                   ("layout_scatter", "scan + scatter")]


def _all_counter_rows(d):
    import csv
    import glob

    out = []
    for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(fn)):
            out.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])))
    return out


def summarize_counters(dirs, out, command):
    """Per-launch counter averages per kernel, and what follows from them:
    the mean L2 read latency seen by the L1s (latency sum / requests), the
    mean number of L2 reads in flight per CU (latency sum / (CUs x cycles))
    and each unit's busy or stall share of a CU's cycles. Cycles per launch
    are GRBM_GUI_ACTIVE / accelerator dies (it is summed over them)."""
    avg = {}
    for d in dirs:
        rows = _all_counter_rows(d)
        for key, _ in COUNTER_KERNELS:
            for c in sorted({c for n, c, _ in rows if key in n}):
                v = [x for n, cc, x in rows if key in n and cc == c]
                avg[(key, c)] = sum(v) / len(v)
    counters = sorted({c for _, c in avg})
    lines = ["# Hardware counters per launch: gate GEMM, selection, scan + scatter", "",
             "Commands (from /tmp, TMPDIR=/tmp; R = repository root), one counter group per run:",
             "", "```", command, "```", "",
             "| counter | " + " | ".join(lab for _, lab in COUNTER_KERNELS) + " |",
             "|---|" + "---|" * len(COUNTER_KERNELS)]
    for c in counters:
        cells = [f"{avg[(k, c)]:,.0f}" if (k, c) in avg else "—" for k, _ in COUNTER_KERNELS]
        lines.append(f"| {c} | " + " | ".join(cells) + " |")

    def derived(k):
        g = lambda c: avg.get((k, c))  # noqa: E731
        cyc = g("GRBM_GUI_ACTIVE")
        res = []
        if cyc:
            cyc /= N_XCD
            res.append(("cycles per launch (per die)", f"{cyc:,.0f}"))
        req, lat = g("TCP_TCC_READ_REQ_sum"), g("TCP_TCC_READ_REQ_LATENCY_sum")
        if req and lat:
            res.append(("L2 read latency, mean (cycles)", f"{lat / req:.0f}"))
            if cyc:
                res.append(("L2 reads in flight per CU, mean", f"{lat / (N_CU * cyc):.0f}"))
        mops, busy = g("SQ_INSTS_VALU_MFMA_MOPS_BF16"), g("SQ_VALU_MFMA_BUSY_CYCLES")
        if mops and cyc:
            # one MOPS unit is 512 flop; time at the 2.4 GHz peak clock
            res.append(("bf16 matrix flop per launch", f"{mops * 512:.4g}"))
            res.append(("bf16 matrix rate at 2.4 GHz (TFLOP/s)",
                        f"{mops * 512 / (cyc / 2.4e9) / 1e12:.0f}"))
        if busy is not None and cyc:
            res.append(("matrix cores busy (share of SIMD cycles)",
                        f"{100 * busy / (N_CU * 4 * cyc):.0f} %"))
        hit, miss = g("TCC_HIT_sum"), g("TCC_MISS_sum")
        if hit is not None and miss:
            res.append(("L2 hit rate", f"{100 * hit / (hit + miss):.1f} %"))
        if cyc:
            for c, lab in (("TA_TA_BUSY_sum", "TA busy"),
                           ("TA_ADDR_STALLED_BY_TC_CYCLES_sum", "TA stalled by the L1"),
                           ("TD_TD_BUSY_sum", "TD busy"),
                           ("TD_TC_STALL_sum", "TD waiting for the L1"),
                           ("TCP_PENDING_STALL_CYCLES_sum", "L1 stalled on pending L2 data"),
                           ("TCP_UTCL1_STALL_INFLIGHT_MAX_sum",
                            "L1 stalled at the translation in-flight limit")):
                if g(c) is not None:
                    res.append((lab + " (share of CU cycles)", f"{100 * g(c) / (N_CU * cyc):.0f} %"))
        return res

    lines += ["", "Derived (MI355X: 256 CUs on 8 dies):", "",
              "| figure | " + " | ".join(lab for _, lab in COUNTER_KERNELS) + " |",
              "|---|" + "---|" * len(COUNTER_KERNELS)]
    per = {k: dict(derived(k)) for k, _ in COUNTER_KERNELS}
    names = []
    for k, _ in COUNTER_KERNELS:
        for n, _ in derived(k):
            if n not in names:
                names.append(n)
    for n in names:
        lines.append(f"| {n} | " + " | ".join(per[k].get(n, "—") for k, _ in COUNTER_KERNELS) + " |")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")


# kernels of one route call of the 16k-token batch
STEP_KERNELS = ("gate_gemm", "route_rows", "layout_scatter", "zero_ints", "route_fused",
                "route_small", "route_layer")


def summarize_traffic(fetch_dir, write_dir, out, command):
    """HBM bytes per launch of the gate GEMM, and per route call (every
    kernel of the call: the sum of each kernel's launches divided by the
    calls), from FETCH_SIZE / WRITE_SIZE runs of `bench.py --route-only
    --copy-probe`, each counter scaled by what it reads for a 1 GiB copy."""
    res = {"gate_gemm_sha256_16": gemm_source_hash(), "sources_sha256_16": all_source_hash(),
           "command": command}
    for key, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _counter_rows(d, counter)
        gemm = [v for n, v in rows if "gate_gemm" in n]
        copy = [v for n, v in rows if "copyBuffer" in n or "copy" in n.lower()]
        res[f"{key}_kib_per_launch"] = sum(gemm) / len(gemm)
        res[f"{key}_kib_copy_1gib"] = max(copy)
        # counter units: KiB; scale by what the counter reads for a known 1 GiB copy
        res[f"{key}_scale"] = COPY_BYTES / (max(copy) * 1024.0)
        calls = len(gemm) or len([v for n, v in rows if "route_fused" in n])
        res[f"{key}_kib_per_step"] = sum(v for n, v in rows
                                         if any(k in n for k in STEP_KERNELS)) / calls
    res["bytes_per_launch"] = (res["fetch_kib_per_launch"] * 1024.0 * res["fetch_scale"] +
                               res["write_kib_per_launch"] * 1024.0 * res["write_scale"])
    res["bytes_per_step"] = (res["fetch_kib_per_step"] * 1024.0 * res["fetch_scale"] +
                             res["write_kib_per_step"] * 1024.0 * res["write_scale"])
    with open(out, "w") as f:
        json.dump(res, f, indent=1)
        f.write("\n")


class HipEvents:
    """hipEvent_t pairs for timing one kernel inside the stream order."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = []
        self.extra = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(a)) == 0
            assert self.hip.hipEventCreate(ctypes.byref(b)) == 0
            self.pairs.append((a, b))

    def plain(self):
        """An event without timing (cheap), for stream-to-stream ordering."""
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        e = ctypes.c_void_p()
        assert self.hip.hipEventCreateWithFlags(ctypes.byref(e), 0x2) == 0  # hipEventDisableTiming
        self.extra.append(e)
        return e

    def record(self, e, stream):
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        assert self.hip.hipEventRecord(e, ctypes.c_void_p(stream.cuda_stream)) == 0

    def elapsed_ms(self, i):
        ms = ctypes.c_float()
        a, b = self.pairs[i]
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def close(self):
        for a, b in self.pairs:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)
        for e in self.extra:
            self.hip.hipEventDestroy(e)


def gemm_source_hash():
    h = hashlib.sha256()
    for path in GEMM_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def all_source_hash():
    """Hash of every kernel and host source of the library."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "top_expert_routing_gate_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per gate-GEMM launch and per route call from the committed
    counter summary, each only if it was taken on the current sources (the
    GEMM's own, or all of them for the whole call); else None."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None, None
    gemm = t.get("bytes_per_launch") if t.get("gate_gemm_sha256_16") == gemm_source_hash() else None
    step = t.get("bytes_per_step") if t.get("sources_sha256_16") == all_source_hash() else None
    return gemm, step


CPU_BASELINE_RUNS = 3  # whole-batch runs at all cores; the median is reported


def _oracle_stages(oracle, wl, x, W, b0):
    """One whole batch through the oracle, stage by stage (the order of the
    path): affinities; scores, selection, weights and entropies; layout; load
    statistics and bias update. Returns seconds per stage."""
    t = {}
    t0 = time.perf_counter()
    h = oracle.affinities(x, W, None)
    t1 = time.perf_counter()
    s64 = oracle.scores(h, wl.score_fn)
    s32 = s64.astype("float32")
    idx, _, _, _ = oracle.select(s32, s64, b0, wl.K, wl.n_groups, wl.topk_groups, wl.n_shared)
    oracle.agg_entropy(s64)
    t2 = time.perf_counter()
    counts = oracle.layout(idx, wl.Nb)[0]
    t3 = time.perf_counter()
    oracle.load_stats(counts[:wl.N])
    oracle.bias_update(b0, counts[:wl.N], 1e-3)
    t4 = time.perf_counter()
    t["gemm"], t["score_select"], t["layout"], t["stats_bias"] = t1 - t0, t2 - t1, t3 - t2, t4 - t3
    t["total"] = t4 - t0
    return t


def cpu_baseline(wl, inp):
    """The oracle, as it stands, on the whole batch: the median of
    CPU_BASELINE_RUNS runs at all host cores, with the time of each stage,
    and one run at one core."""
    import oracle

    x = inp["x"][0].float().numpy()
    W = inp["W"][0].float().numpy()
    b0 = inp["bias"][0].numpy()
    cores = oracle.num_threads()
    runs = [_oracle_stages(oracle, wl, x, W, b0) for _ in range(CPU_BASELINE_RUNS)]
    med = {k: statistics.median(r[k] for r in runs) for k in runs[0]}
    oracle.set_num_threads(1)
    try:
        one = _oracle_stages(oracle, wl, x, W, b0)
    finally:
        oracle.set_num_threads(cores)
    return {"value": wl.T / med["total"], "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the whole batch ({wl.T} tokens, d={wl.d}, N={wl.N}), median of "
                      f"{CPU_BASELINE_RUNS} runs at {cores} threads: fp64 affinities, scores, "
                      "selection, entropies, layout, load statistics, bias update",
            "stages_ms": {k: v * 1e3 for k, v in med.items()},
            "one_core": {"value": wl.T / one["total"], "cores": 1, "runs": 1,
                         "stages_ms": {k: v * 1e3 for k, v in one.items()}}}


def time_dispatch_combine(moer, torch, wl, x, outs, stream, steps):
    """Local dispatch of the batch to its experts and the weighted combine
    back, on the route's last layout (bf16 rows; the dispatched rows stand in
    for the expert outputs). Each is timed over `steps` launches between two
    events on the route's stream. Algorithmic bytes per launch: every token
    row read once and written Kt times (dispatch), Kt rows read and one
    written (combine): L*T*(1+Kt)*d*2."""
    L, T, Kt, d = wl.n_layers, wl.T, wl.Kt, wl.d
    dev = x.device
    xd = torch.empty(L, T * Kt, d, dtype=torch.bfloat16, device=dev)
    y = torch.empty(L, T, d, dtype=torch.bfloat16, device=dev)
    inv, w = outs["inv_perm"], outs["topk_w"]
    res = {}
    with torch.cuda.stream(stream):
        for _ in range(3):
            moer.dispatch(x, inv, Kt, out=xd)
            moer.combine(xd, w, inv, out=y)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        for _ in range(steps):
            moer.dispatch(x, inv, Kt, out=xd)
        ev[1].record(stream)
        for _ in range(steps):
            moer.combine(xd, w, inv, out=y)
        ev[2].record(stream)
    torch.cuda.synchronize()
    nbytes = L * T * (1 + Kt) * d * 2
    for k, (a, b) in (("dispatch", (0, 1)), ("combine", (1, 2))):
        us = ev[a].elapsed_time(ev[b]) * 1e3 / steps
        gbs = nbytes / (us * 1e-6) / 1e9
        res[k] = {"us": us, "bytes": nbytes, "achieved": gbs, "peak": HBM_PEAK_GBS,
                  "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS}
    del xd, y
    return res


def time_forcible_layout(moer, torch, wl, outs, stream, steps):
    """The layout path (moer_route in INDICES mode: counts, offsets, perm,
    inv_perm) on the batch's routed ids and on forcibly balanced ids (every
    expert T*K/N assignments), each over `steps` calls between two events on
    the route's stream: the balanced case is the upper bound the pages'
    forcible balancing measures."""
    L, T, K, N, ns = wl.n_layers, wl.T, wl.K, wl.N, wl.n_shared
    dev = outs["topk_idx"].device
    desc = moer.make_desc(n_layers=L, T=T, N=N, K=K, n_shared=ns, input=moer.MOER_IN_INDICES)
    i32 = dict(dtype=torch.int32, device=dev)
    Kt, Nb = K + ns, N + ns
    lay = dict(counts=torch.empty(L, Nb, **i32), offsets=torch.empty(L, Nb + 1, **i32),
               perm=torch.empty(L, T * Kt, **i32), inv_perm=torch.empty(L, T * Kt, **i32))
    ws = torch.empty(max(1, moer.moer_route_workspace_bytes(desc)), dtype=torch.uint8, device=dev)
    with torch.cuda.stream(stream):
        balanced = moer.balanced_indices(T, K, N, n_layers=L, n_shared=ns, device=dev)
        routed = outs["topk_idx"].clone()
        res = {}
        for name, ids in (("routed_ids", routed), ("balanced_ids", balanced)):
            call = moer.PreparedRoute(desc, workspace=ws, idx_in=ids, **lay)
            for _ in range(3):
                call()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            for _ in range(steps):
                call()
            ev[1].record(stream)
            torch.cuda.synchronize()
            res[name] = {"us": ev[0].elapsed_time(ev[1]) * 1e3 / steps,
                         "max_count": int(lay["counts"][:, :N].max())}
    return res


def time_capacity(moer, torch, wl, x, Wd, bias, stream, steps):
    """The route with the pages' capacity (1.25 x T*K/N) on the batch, and on
    the same batch with the collapse workload's celebrity offset (+3.0 on
    experts 2, 4, 7, 12), each over `steps` calls between two events on the
    route's stream (bias not updated, so every call is the same work)."""
    L, T, N, K = wl.n_layers, wl.T, wl.N, wl.K
    cap = moer.expert_capacity(T, K, N)
    dev = x.device
    i32, f32 = dict(dtype=torch.int32, device=dev), dict(dtype=torch.float32, device=dev)
    Kt, Nb = wl.Kt, wl.Nb
    bufs = dict(topk_idx=torch.empty(L, T, Kt, **i32), topk_w=torch.empty(L, T, Kt, **f32),
                tok_entropy=torch.empty(L, T, **f32), agg_entropy=torch.empty(L, **f32),
                counts=torch.empty(L, Nb, **i32), offsets=torch.empty(L, Nb + 1, **i32),
                perm=torch.empty(L, T * Kt, **i32), inv_perm=torch.empty(L, T * Kt, **i32),
                cap_stats=torch.empty(L, 2, **i32))
    desc = moer.make_desc(n_layers=L, T=T, d=wl.d, N=N, K=K, n_groups=wl.n_groups,
                          topk_groups=wl.topk_groups, n_shared=wl.n_shared, score_fn=wl.score_fn,
                          dtype=wl.dtype, capacity=cap)
    ws = torch.empty(moer.moer_route_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    celeb = torch.zeros(N, **f32)
    celeb[[2, 4, 7, 12]] = 3.0
    res = {"capacity": cap}
    with torch.cuda.stream(stream):
        for name, off in (("dsv3_group", None), ("collapse_offsets", celeb)):
            call = moer.PreparedRoute(desc, workspace=ws, x=x, w_gate=Wd, bias=bias,
                                      logit_offset=off, **bufs)
            for _ in range(3):
                call()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            for _ in range(steps):
                call()
            ev[1].record(stream)
            torch.cuda.synchronize()
            st = bufs["cap_stats"][0].tolist()
            res[name] = {"us": ev[0].elapsed_time(ev[1]) * 1e3 / steps, "rerouted": st[0],
                         "dropped": st[1], "max_count": int(bufs["counts"][:, :N].max())}
    del ws
    return res


def time_balance_step(moer, torch, wl, outs, stream, steps):
    """The balancing-rule variants on the batch's counts, each over `steps`
    calls between two events on the route's stream (a copy of the bias, so
    the route's own bias is untouched)."""
    dev = outs["counts"].device
    res = {}
    with torch.cuda.stream(stream):
        for name, kw in (("sign", dict(rule="sign", step=1e-3)),
                         ("proportional_ema_every4", dict(rule="proportional", step=0.05,
                                                          alpha=0.1, every=4))):
            bias = torch.zeros(wl.n_layers, wl.N, device=dev)
            state = moer.BalanceState(wl.n_layers, wl.N, device=dev)
            for _ in range(3):
                moer.balance_step(bias, outs["counts"], state=state, **kw)
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            for _ in range(steps):
                moer.balance_step(bias, outs["counts"], state=state, **kw)
            ev[1].record(stream)
            torch.cuda.synchronize()
            res[name] = {"us": ev[0].elapsed_time(ev[1]) * 1e3 / steps}
    return res


# ---------------------------------------------------------------- report
HBM_PEAK_BPS = HBM_PEAK_GBS * 1e9
# MFMA_BF16_PEAK (above) also bounds fp32 inputs here


def algorithmic_bytes(wl):
    """Bytes a route call must move: x, W_g and bias read; ids, weights, perm
    (Kt x 12 B per token), counts, offsets and per-token entropy written."""
    es = 2 if wl.dtype == 0 else 4
    L, T, N, d, Kt, Nb = wl.n_layers, wl.T, wl.N, wl.d, wl.Kt, wl.Nb
    return L * (T * d * es + N * d * es + N * 4 + T * Kt * 12 + Nb * 4 + (Nb + 1) * 4 + T * 4)


def _pct(v, q):
    v = sorted(v)
    return v[min(len(v) - 1, max(0, int(round(q * (len(v) - 1)))))]


def _clocks():
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=30)
        keep = [l.strip() for l in r.stdout.splitlines() if "sclk" in l or "mclk" in l]
        return keep[:4] or ["(rocm-smi printed no clock lines)"]
    except (OSError, subprocess.SubprocessError) as exc:
        return [f"(rocm-smi unavailable: {exc})"]


def run_report(args):
    import statistics

    import torch

    import oracle
    import top_expert_routing_gate_amd as moer
    import workloads

    dev = torch.device("cuda:0")
    out = ["# Router on every workload shape (one MI355X)", "",
           f"Command: `python bench.py --report {args.out_report}` (from the repository root).",
           "", "Clocks before: " + "; ".join(_clocks()), ""]
    # read (not written) between calls: evicts the 256 MB last-level cache
    # without leaving dirty lines to write back inside the next timed call
    flush = torch.ones(256 << 20, dtype=torch.float16, device=dev)  # 512 MB
    stream = torch.cuda.Stream()
    ev = HipEvents(400)
    empty = []
    for i in range(200):
        ev.record(ev.pairs[i][0], stream)
        ev.record(ev.pairs[i][1], stream)
    torch.cuda.synchronize()
    empty = [ev.elapsed_ms(i) * 1e3 for i in range(200)]
    pair_us = statistics.median(empty)
    out += [f"An empty event pair reads {pair_us:.2f} us (median of 200); the per-call times "
            "below are the event-bracketed medians less that.", "",
            "| workload | L x T | reps | median us | p10 | p90 | gate GEMM us (median) | routed tokens/s "
            "| roofline us | % of roofline | oracle tokens/s (all cores) | oracle tokens/s (1 core) |",
            "|---|---|---|---|---|---|---|---|---|---|---|---|"]
    graph_rows = []
    order = ["tiny_softmax", "mixtral_top2", "dsv3_group", "collapse_balance", "decode_layers"]
    for name in order:
        wl = workloads.WORKLOADS[name]
        print(f"[report] {name}: inputs", file=sys.stderr, flush=True)
        W, b0, off, gen = workloads.make_router(wl)
        x = workloads.make_hidden(wl, gen=gen)
        L, T, N, Kt, Nb = wl.n_layers, wl.T, wl.N, wl.Kt, wl.Nb
        xd, Wd = x.to(dev), W.to(dev)
        bias = b0.clone().to(dev)
        offd = None if off is None else off.to(dev)
        desc = moer.make_desc(n_layers=L, T=T, d=wl.d, N=N, K=wl.K, n_groups=wl.n_groups,
                              topk_groups=wl.topk_groups, n_shared=wl.n_shared,
                              score_fn=wl.score_fn, dtype=wl.dtype)
        i32, f32 = dict(dtype=torch.int32, device=dev), dict(dtype=torch.float32, device=dev)
        outs = dict(topk_idx=torch.empty(L, T, Kt, **i32), topk_w=torch.empty(L, T, Kt, **f32),
                    tok_entropy=torch.empty(L, T, **f32), agg_entropy=torch.empty(L, **f32),
                    counts=torch.empty(L, Nb, **i32), offsets=torch.empty(L, Nb + 1, **i32),
                    perm=torch.empty(L, T * Kt, **i32), inv_perm=torch.empty(L, T * Kt, **i32))
        stats = torch.empty(L, 64, dtype=torch.uint8, device=dev)
        ws = torch.empty(max(1, moer.moer_route_workspace_bytes(desc)), dtype=torch.uint8,
                         device=dev)
        call = moer.PreparedRoute(desc, workspace=ws, stream=stream, x=xd, w_gate=Wd, bias=bias,
                                  logit_offset=offd, load_stats=stats, bias_update=bias,
                                  bias_update_u=1e-3, **outs)
        reps = 50 if T * L >= 16384 else 200
        # warm-up: calls until the clocks are steady, then 10 more
        clock_ramp(torch, call)
        for _ in range(10):
            call()
        torch.cuda.synchronize()
        times, gemm = [], []
        for i in range(reps):
            with torch.cuda.stream(stream):
                # the last-level cache holds none of the inputs; on the route's
                # stream, outside the events
                flush.max()
            ev.record(ev.pairs[i][0], stream)
            call()
            ev.record(ev.pairs[i][1], stream)
        torch.cuda.synchronize()
        times = [ev.elapsed_ms(i) * 1e3 - pair_us for i in range(reps)]
        for i in range(reps):
            with torch.cuda.stream(stream):
                flush.max()
            call(ev.pairs[i][0], ev.pairs[i][1])
        torch.cuda.synchronize()
        gemm = [ev.elapsed_ms(i) * 1e3 - pair_us for i in range(reps)]
        med = statistics.median(times)
        t_roof = max(algorithmic_bytes(wl) / HBM_PEAK_BPS, 2.0 * L * T * N * wl.d / MFMA_BF16_PEAK)
        # oracle: one layer (bounded sample at one core)
        print(f"[report] {name}: oracle", file=sys.stderr, flush=True)
        xs = x[0].float().numpy()
        Ws = W[0].float().numpy()
        bs = b0[0].numpy()
        osel = None if off is None else off.numpy()

        def oracle_rate(ntok):
            t0 = time.perf_counter()
            o = oracle.route(x=xs[:ntok], W=Ws, offset=osel, bias=bs, K=wl.K,
                             score_fn=wl.score_fn, n_groups=wl.n_groups,
                             topk_groups=wl.topk_groups, n_shared=wl.n_shared)
            oracle.load_stats(o["counts"][:N])
            oracle.bias_update(bs, o["counts"][:N], 1e-3)
            return ntok / (time.perf_counter() - t0)

        all_cores = oracle.num_threads()
        r_all = oracle_rate(T)
        oracle.set_num_threads(1)
        r_one = oracle_rate(min(T, 1024))
        oracle.set_num_threads(all_cores)
        out.append(f"| {name} | {L} x {T} | {reps} | {med:.1f} | {_pct(times, 0.1):.1f} | "
                   f"{_pct(times, 0.9):.1f} | {statistics.median(gemm):.1f} | "
                   f"{L * T / (med * 1e-6) / 1e6:.1f} M | {t_roof * 1e6:.2f} | "
                   f"{100 * t_roof / (med * 1e-6):.1f} | {r_all / 1e3:.1f} k ({all_cores}) | "
                   f"{r_one / 1e3:.2f} k |")
        if name in ("tiny_softmax", "mixtral_top2", "decode_layers"):
            graph_rows += graph_timing(moer, torch, wl, desc, xd, Wd, b0.to(dev), offd, ev,
                                       pair_us, stream)
        del xd, Wd, ws, outs
    out += ["", "Oracle: one layer's batch at all cores (one core: the first min(T, 1024) "
            "tokens), including load statistics and the bias update.", "",
            "## HIP graph replay", "",
            "The route call (no bias update, so replays repeat the same work) captured once "
            "and replayed; every replay's outputs equal the eager call's. Host: time to "
            "submit one call (200 in a row, no synchronisation). GPU: time per call of 200 "
            "calls run back to back (queued behind a spin kernel, so the host cost is "
            "hidden). Paired: one call between an event pair, the pairs queued behind the "
            "spin (median, less an empty pair). Alone: the same with the host waiting for "
            "each call to finish before submitting the next (median, less an empty pair).",
            "",
            "| case | host us eager | host us graph | GPU us/call eager | GPU us/call graph "
            "| paired us eager | paired us graph | alone us eager | alone us graph |",
            "|---|---|---|---|---|---|---|---|---|"] + graph_rows
    out += ["", "## Collapse workload: 100 balancing iterations", ""] + collapse_series(
        moer, torch, workloads, ev, pair_us, stream)
    out += ["", "Clocks after: " + "; ".join(_clocks())]
    ev.close()
    with open(args.out_report, "w") as f:
        f.write("\n".join(out) + "\n")
    print(f"[report] written to {args.out_report}", file=sys.stderr, flush=True)


def graph_timing(moer, torch, wl, desc, x, W, bias, off, ev, pair_us, stream):
    """Eager vs HIP-graph replay of one route call (the whole batch, and for
    the layered workload also one layer alone)."""
    import statistics

    rows = []
    cases = [("all layers", desc, x, W, bias)]
    if wl.n_layers > 1:
        d1 = moer.make_desc(n_layers=1, T=wl.T, d=wl.d, N=wl.N, K=wl.K, n_groups=wl.n_groups,
                            topk_groups=wl.topk_groups, n_shared=wl.n_shared,
                            score_fn=wl.score_fn, dtype=wl.dtype)
        cases.append(("one layer", d1, x[:1].contiguous(), W[:1].contiguous(),
                      bias[:1].contiguous()))
    for label, d, xx, WW, bb in cases:
        L, T, Kt, Nb = d.n_layers, d.T, wl.Kt, wl.Nb
        dev = xx.device
        i32, f32 = dict(dtype=torch.int32, device=dev), dict(dtype=torch.float32, device=dev)

        def bufs():
            return dict(topk_idx=torch.empty(L, T, Kt, **i32), topk_w=torch.empty(L, T, Kt, **f32),
                        counts=torch.empty(L, Nb, **i32), offsets=torch.empty(L, Nb + 1, **i32),
                        perm=torch.empty(L, T * Kt, **i32), inv_perm=torch.empty(L, T * Kt, **i32))
        ws = torch.empty(max(1, moer.moer_route_workspace_bytes(d)), dtype=torch.uint8, device=dev)
        eager_out, graph_out = bufs(), bufs()
        eager = moer.PreparedRoute(d, workspace=ws, stream=stream, x=xx, w_gate=WW, bias=bb,
                                   logit_offset=off, **eager_out)
        gs = torch.cuda.Stream()
        ws2 = torch.empty_like(ws)
        cap = moer.PreparedRoute(d, workspace=ws2, stream=gs, x=xx, w_gate=WW, bias=bb,
                                 logit_offset=off, **graph_out)
        for _ in range(3):
            eager()
        with torch.cuda.stream(gs):
            for _ in range(3):
                cap()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gs):
            cap()
        torch.cuda.synchronize()
        reps = 200
        for _ in range(50):
            eager()
        torch.cuda.synchronize()
        res = {}
        with torch.cuda.stream(stream):
            for kind, fn in (("eager", eager), ("graph", g.replay)):
                # host time to submit one call (no synchronisation in between)
                t0 = time.perf_counter()
                for _ in range(reps):
                    fn()
                host = (time.perf_counter() - t0) / reps * 1e6
                torch.cuda.synchronize()
                # GPU time per call: the stream is held by a spin kernel long
                # enough for the host to queue every call first, so the
                # calls run back to back whatever the host cost
                spin = int(2.4e3 * (2.0 * host * reps + 2000.0))  # ~2.4 GHz shader clock
                torch.cuda._sleep(spin)
                ev.record(ev.pairs[0][0], stream)
                for _ in range(reps):
                    fn()
                ev.record(ev.pairs[0][1], stream)
                torch.cuda.synchronize()
                b2b = ev.elapsed_ms(0) * 1e3 / reps
                # one call between an event pair, each pair queued behind the
                # spin as well
                torch.cuda._sleep(spin)
                for i in range(reps):
                    ev.record(ev.pairs[i][0], stream)
                    fn()
                    ev.record(ev.pairs[i][1], stream)
                torch.cuda.synchronize()
                paired = statistics.median(ev.elapsed_ms(i) * 1e3 - pair_us for i in range(reps))
                # the same pairs with the host submitting each call after the
                # previous one has finished (what a single call sees)
                alone = []
                for i in range(50):
                    ev.record(ev.pairs[i][0], stream)
                    fn()
                    ev.record(ev.pairs[i][1], stream)
                    torch.cuda.synchronize()
                    alone.append(ev.elapsed_ms(i) * 1e3 - pair_us)
                res[kind] = (host, b2b, paired, statistics.median(alone))
        for k in eager_out:
            assert torch.equal(eager_out[k], graph_out[k]), f"graph replay differs: {k}"
        e, gr = res["eager"], res["graph"]
        rows.append(f"| {wl.name}, {label} ({L} x {T}) | {e[0]:.1f} | {gr[0]:.1f} | {e[1]:.1f} | "
                    f"{gr[1]:.1f} | {e[2]:.1f} | {gr[2]:.1f} | {e[3]:.1f} | {gr[3]:.1f} |")
        del g
    return rows


def collapse_series(moer, torch, workloads, ev, pair_us, stream):
    """The collapse workload (celebrity offsets +3.0 on experts 2, 4, 7, 12)
    routed 100 times with the fused sign-step bias update (u = 1e-3); x of
    iteration i is drawn on the GPU from seed 1000 + i (the CPU recipe's 100
    draws of 235 MB would take minutes)."""
    import statistics

    wl = workloads.WORKLOADS["collapse_balance"]
    dev = torch.device("cuda:0")
    W, b0, off, _ = workloads.make_router(wl)
    Wd, bias, offd = W.to(dev), b0.clone().to(dev), off.to(dev)
    L, T, N, Kt, Nb = wl.n_layers, wl.T, wl.N, wl.Kt, wl.Nb
    desc = moer.make_desc(n_layers=L, T=T, d=wl.d, N=N, K=wl.K, n_groups=wl.n_groups,
                          topk_groups=wl.topk_groups, score_fn=wl.score_fn, dtype=wl.dtype)
    i32, f32 = dict(dtype=torch.int32, device=dev), dict(dtype=torch.float32, device=dev)
    outs = dict(topk_idx=torch.empty(L, T, Kt, **i32), topk_w=torch.empty(L, T, Kt, **f32),
                counts=torch.empty(L, Nb, **i32), offsets=torch.empty(L, Nb + 1, **i32),
                perm=torch.empty(L, T * Kt, **i32))
    stats = torch.empty(L, 64, dtype=torch.uint8, device=dev)
    ws = torch.empty(moer.moer_route_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    x = torch.empty(L, T, wl.d, dtype=torch.bfloat16, device=dev)
    call = moer.PreparedRoute(desc, workspace=ws, stream=stream, x=x, w_gate=Wd, bias=bias,
                              logit_offset=offd, load_stats=stats, bias_update=bias,
                              bias_update_u=1e-3, **outs)
    rows = ["| iteration | imbalance (max/mean) | load entropy (bits) | celebrity share | "
            "route us |", "|---|---|---|---|---|"]
    celeb = list(wl.celebrities)
    times = []
    for i in range(100):
        g = torch.Generator(device=dev).manual_seed(1000 + i)
        x.copy_(torch.randn(L, T, wl.d, generator=g, device=dev).to(torch.bfloat16))
        torch.cuda.synchronize()
        ev.record(ev.pairs[0][0], stream)
        call()
        ev.record(ev.pairs[0][1], stream)
        torch.cuda.synchronize()
        times.append(ev.elapsed_ms(0) * 1e3 - pair_us)
        st = moer.decode_load_stats(stats.cpu())[0]
        c = outs["counts"][0, :N].cpu()
        share = float(c[celeb].sum()) / max(1, int(c.sum()))
        if i % 10 == 0 or i == 99:
            rows.append(f"| {i} | {st['imbalance']:.3f} | {st['h_load_bits']:.3f} | "
                        f"{share:.3f} | {times[-1]:.1f} |")
        if i % 25 == 0:
            print(f"[report] collapse iteration {i}", file=sys.stderr, flush=True)
    rows += ["", f"Median route call over the 100 iterations: {statistics.median(times):.1f} us "
             "(bias updated in place by the same call)."]
    return rows


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, args.command, args.steps, args.warmup)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.out, args.command)
        return
    if args.summarize_stages:
        summarize_stages(*args.summarize_stages, args.out, args.command)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.out, args.command)
        return
    if args.report:
        args.out_report = args.report
        run_report(args)
        return
    if args.stage_run:
        run_stage_calls(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the router is measured "
              "at one GPU's share; multi-GPU sharding is a design note, not built.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import top_expert_routing_gate_amd as moer
    import workloads

    wl = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    print(f"[bench] generating inputs for {wl.name}", file=sys.stderr, flush=True)
    W, b0, off, gen = workloads.make_router(wl)
    xs_cpu = [workloads.make_hidden(wl, gen=gen)]
    xs_cpu += [workloads.make_hidden(wl, seed=wl.seed + 1 + i) for i in range(2)]
    xs = [x.to(dev) for x in xs_cpu]
    Wd, bias = W.to(dev), b0.clone().to(dev)
    offd = None if off is None else off.to(dev)
    L, T, N, Kt, Nb = wl.n_layers, wl.T, wl.N, wl.Kt, wl.Nb
    desc = moer.make_desc(n_layers=L, T=T, d=wl.d, N=N, K=wl.K, n_groups=wl.n_groups,
                          topk_groups=wl.topk_groups, n_shared=wl.n_shared,
                          score_fn=wl.score_fn, dtype=wl.dtype, input=moer.MOER_IN_HIDDEN)
    i32, f32 = dict(dtype=torch.int32, device=dev), dict(dtype=torch.float32, device=dev)
    outs = dict(topk_idx=torch.empty(L, T, Kt, **i32), topk_w=torch.empty(L, T, Kt, **f32),
                tok_entropy=torch.empty(L, T, **f32), agg_entropy=torch.empty(L, **f32),
                counts=torch.empty(L, Nb, **i32), offsets=torch.empty(L, Nb + 1, **i32),
                perm=torch.empty(L, T * Kt, **i32), inv_perm=torch.empty(L, T * Kt, **i32))
    stats = torch.empty(L, 64, dtype=torch.uint8, device=dev)
    ev = HipEvents(args.steps)

    # The router runs on a stream of its own (default priority), as a serving
    # or training loop would (the legacy default stream adds per-launch
    # waits). With --overlap, consecutive steps alternate between two such
    # streams, each with its own workspace: step i+1's gate GEMM reads only x
    # and W_g, so it may overlap step i's selection and layout, while step
    # i+1's selection waits for an event recorded after step i (so it sees
    # step i's bias update; the results are the one-stream sequence).
    nstream = 2 if args.overlap else 1
    streams = [torch.cuda.Stream() for _ in range(nstream)]
    wss = [torch.empty(moer.moer_route_workspace_bytes(desc), dtype=torch.uint8, device=dev)
           for _ in range(nstream)]
    done = [ev.plain() for _ in range(nstream)]
    torch.cuda.synchronize()
    # arguments marshalled once per (stream, x batch); the loop only enqueues
    calls = []
    for k in range(nstream):
        with torch.cuda.stream(streams[k]):
            calls.append([moer.PreparedRoute(desc, workspace=wss[k], x=xb, w_gate=Wd, bias=bias,
                                             logit_offset=offd, load_stats=stats,
                                             bias_update=bias, bias_update_u=1e-3, **outs)
                          for xb in xs])

    def step(i, events=None):
        k = i % nstream
        wait = done[(i - 1) % nstream] if (nstream > 1 and i > 0) else None
        calls[k][i % len(xs)](*(events or (None, None)), ev_select_wait=wait)
        if nstream > 1:  # only the overlapped schedule chains steps through events
            ev.record(done[k], streams[k])

    def sync_streams():
        # every stream has reached the end of what was enqueued so far
        for st in streams:
            st.synchronize()

    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        bcopy = torch.empty_like(a)
        bcopy.copy_(a)
        torch.cuda.synchronize()
        del a, bcopy
    for i in range(args.warmup):
        step(i)
    sync_streams()
    torch.cuda.synchronize()
    ramp_i = [args.warmup]

    def ramp_step():
        step(ramp_i[0])
        ramp_i[0] += 1

    n_ramp = clock_ramp(torch, ramp_step)
    print(f"[bench] warmup done ({args.warmup} steps, then {n_ramp} more over "
          f"{CLOCK_RAMP_S * 1e3:.0f} ms for the clocks); timing {args.steps} steps",
          file=sys.stderr, flush=True)
    # timed region 1 (value): K uninstrumented steps between two barriers; the
    # start event is on the first step's stream (the other stream's first
    # work waits for step 0 through the chain of events anyway), the end event
    # after every stream has finished
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    i0 = args.warmup
    t_wall = time.perf_counter()
    e0.record(streams[i0 % nstream])
    for st in streams:
        if st is not streams[i0 % nstream]:
            st.wait_event(e0)
    for i in range(args.steps):
        step(i0 + i)
    last = streams[(i0 + args.steps - 1) % nstream]
    for st in streams:
        if st is not last:
            last.wait_stream(st)
    e1.record(last)
    sync_streams()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = e0.elapsed_time(e1) / args.steps
    # timed region 2 (dominant kernel): the same K steps, the gate GEMM's
    # launch recording an event pair at the kernel's own start and end
    # (hipExtLaunchKernel: the dispatch's timestamps, as a kernel trace reads
    # them); the events stay out of region 1
    for i in range(args.steps):
        step(args.warmup + args.steps + i, ev.pairs[i])
    sync_streams()
    torch.cuda.synchronize()
    gemm_us = [ev.elapsed_ms(i) * 1e3 for i in range(args.steps)]
    gemm_ms = statistics.mean(gemm_us) * 1e-3
    ev.close()
    st = moer.decode_load_stats(stats.cpu())[0]
    print(f"[bench] {ms_step * 1e3:.1f} us/step (wall {t_wall / args.steps * 1e6:.1f} us), "
          f"gate GEMM {gemm_ms * 1e3:.1f} us (mean; median {statistics.median(gemm_us):.1f}, "
          f"min {min(gemm_us):.1f}); last imbalance {st['imbalance']:.3f}", file=sys.stderr,
          flush=True)

    dc = None
    if args.route_only:
        args.no_dispatch_combine = args.no_forcible = True
    if not args.no_dispatch_combine:
        dc = time_dispatch_combine(moer, torch, wl, xs[0], outs, streams[0], args.steps)
        print(f"[bench] dispatch {dc['dispatch']['us']:.1f} us, combine "
              f"{dc['combine']['us']:.1f} us", file=sys.stderr, flush=True)

    fl = None
    if not args.no_forcible:
        fl = time_forcible_layout(moer, torch, wl, outs, streams[0], args.steps)
        print(f"[bench] layout (INDICES mode): routed ids {fl['routed_ids']['us']:.1f} us, "
              f"balanced ids {fl['balanced_ids']['us']:.1f} us", file=sys.stderr, flush=True)

    cp = bs = None
    if not args.route_only:
        cp = time_capacity(moer, torch, wl, xs[0], Wd, bias, streams[0], args.steps)
        print(f"[bench] capacity {cp['capacity']}: {cp['dsv3_group']['us']:.1f} us "
              f"({cp['dsv3_group']['rerouted']} rerouted), with celebrity offsets "
              f"{cp['collapse_offsets']['us']:.1f} us ({cp['collapse_offsets']['rerouted']} rerouted, "
              f"{cp['collapse_offsets']['dropped']} dropped)", file=sys.stderr, flush=True)
        bs = time_balance_step(moer, torch, wl, outs, streams[0], args.steps)
        print(f"[bench] balance step: sign {bs['sign']['us']:.1f} us, proportional+EMA "
              f"{bs['proportional_ema_every4']['us']:.1f} us", file=sys.stderr, flush=True)

    esize = 2 if wl.dtype == workloads.BF16 else 4
    gemm_bytes = L * (T + N) * wl.d * esize  # x + W_g of every layer per launch
    gemm_achieved = gemm_bytes / (gemm_ms * 1e-3) / 1e9
    step_bytes = algorithmic_bytes(wl)
    step_achieved = step_bytes / (ms_step * 1e-3) / 1e9
    gemm_traffic, step_traffic = measured_traffic()
    line = {
        "metric": METRIC,
        "value": T * L / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_ramp": {"steps": n_ramp, "ms": CLOCK_RAMP_S * 1e3},
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": T, "hidden": wl.d, "experts": N,
                   "groups": wl.n_groups, "groups_kept": wl.topk_groups, "top_k": wl.K,
                   "score": "sigmoid" if wl.score_fn == 1 else "softmax",
                   "step": "route+load_stats+bias_update (fused)", "x_batches_rotated": len(xs),
                   "streams": nstream},
        # the whole step (every kernel of the route call) against the HBM
        # roofline of its algorithmic bytes; the dominant kernel beside it
        "roofline": {"bound": "hbm", "achieved": step_achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": step_achieved / HBM_PEAK_GBS,
                     "traffic": step_traffic, "scope": "step", "alg_bytes": step_bytes,
                     "kernel": {"name": "gate_gemm", "bound": "hbm", "achieved": gemm_achieved,
                                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                "frac": gemm_achieved / HBM_PEAK_GBS, "traffic": gemm_traffic,
                                "kernel_us": gemm_ms * 1e3,
                                "kernel_us_median": statistics.median(gemm_us),
                                "alg_bytes": gemm_bytes,
                                "timing": "hipExtLaunchKernel events at the kernel's start and "
                                          "end, mean over the K steps"}},
    }
    if dc is not None:
        line["dispatch_combine"] = dc
    if fl is not None:
        line["forcible_layout"] = fl
    if bs is not None:
        line["balance_step"] = bs
    if cp is not None:
        line["capacity_route"] = cp
    if not args.no_cpu_baseline:
        print(f"[bench] timing the CPU oracle: {CPU_BASELINE_RUNS} whole batches at all cores, "
              "one at one core", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl, {"x": xs_cpu[0], "W": W, "bias": b0})
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
