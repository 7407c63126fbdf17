"""Router hot-path benchmark on one MI355X.

One step = one pass of the whole hot path over one batch of the
DeepSeek-V3-style router (16384 tokens, d=7168, 256 experts in 8 groups of
32, keep 4 groups, top-8, sigmoid, selection bias):
  moer_route (gate GEMM, scores, group-limited top-k, weights, per-token and
  batch-mean entropy, counts/offsets/perm/inv_perm, and, fused into the same
  call, the load statistics and the in-place sign-step bias update).
Inputs are resident in HBM before timing; x rotates over three distinct
batches (705 MB in all, larger than the 256 MB last-level cache) so each
step streams its batch from HBM.

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
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
GEMM_SRC = os.path.join(ROOT, "top_expert_routing_gate_amd", "csrc", "gate_gemm.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_gemm_dsv3_traffic.json")
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
    p.add_argument("--no-forcible", action="store_true",
                   help="skip timing the layout on forcibly balanced ids against the routed ids")
    p.add_argument("--copy-probe", action="store_true",
                   help="also run one plain 1 GiB device copy (counter calibration)")
    p.add_argument("--summarize-trace", metavar="DIR",
                   help="write a per-kernel table from a rocprofv3 --kernel-trace --stats dir")
    p.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="calibrated HBM bytes per gate-GEMM launch from two --pmc runs")
    p.add_argument("--command", default="", help="profiling command recorded in a summary")
    p.add_argument("--out", help="output file of a summary")
    return p.parse_args()


COPY_BYTES = 1 << 30


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


def summarize_traffic(fetch_dir, write_dir, out, command):
    res = {"gate_gemm_sha256_16": gemm_source_hash(), "command": command}
    for key, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _counter_rows(d, counter)
        gemm = [v for n, v in rows if "gate_gemm" in n]
        copy = [v for n, v in rows if "copyBuffer" in n or "copy" in n.lower()]
        res[f"{key}_kib_per_launch"] = sum(gemm) / len(gemm)
        res[f"{key}_kib_copy_1gib"] = max(copy)
        # counter units: KiB; scale by what the counter reads for a known 1 GiB copy
        res[f"{key}_scale"] = COPY_BYTES / (max(copy) * 1024.0)
    res["bytes_per_launch"] = (res["fetch_kib_per_launch"] * 1024.0 * res["fetch_scale"] +
                               res["write_kib_per_launch"] * 1024.0 * res["write_scale"])
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
    with open(GEMM_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per gate-GEMM launch from the committed counter summary, if
    it was taken on the current kernel source (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("gate_gemm_sha256_16") != gemm_source_hash():
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(wl, inp):
    """The oracle, as it stands, on one full batch of the workload."""
    import numpy as np

    import oracle

    x = inp["x"][0].float().numpy()
    W = inp["W"][0].float().numpy()
    b = inp["bias"][0].numpy()
    t0 = time.perf_counter()
    out = oracle.route(x=x, W=W, bias=b, K=wl.K, score_fn=wl.score_fn, n_groups=wl.n_groups,
                       topk_groups=wl.topk_groups, n_shared=wl.n_shared)
    oracle.load_stats(out["counts"][:wl.N])
    oracle.bias_update(b, out["counts"][:wl.N], 1e-3)
    dt = time.perf_counter() - t0
    del np
    return {"value": wl.T / dt, "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"one full batch ({wl.T} tokens, d={wl.d}, N={wl.N}): fp64 affinities, "
                      f"scores, selection, entropy, layout, load stats, bias update; {dt:.1f} s"}


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


def main():
    args = parse()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, args.command, args.steps, args.warmup)
        return
    if args.summarize_traffic:
        summarize_traffic(*args.summarize_traffic, args.out, args.command)
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
    print(f"[bench] warmup done ({args.warmup} steps); timing {args.steps} steps",
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
    # timed region 2 (roofline): the same K steps with hipEvents around every
    # gate GEMM launch on the route's stream (events cost a few us per step,
    # so they stay out of region 1)
    for i in range(args.steps):
        step(args.warmup + args.steps + i, ev.pairs[i])
    sync_streams()
    torch.cuda.synchronize()
    event_ms = sum(ev.elapsed_ms(i) for i in range(args.steps)) / args.steps
    # An event pair reads a few us even with nothing between its events (the
    # markers' own processing): measure that on the same stream, the same
    # number of times, and take it off the GEMM's bracketed time. The kernel
    # trace of the same command shows the remainder is the kernel's duration.
    for i in range(args.steps):
        ev.record(ev.pairs[i][0], streams[0])
        ev.record(ev.pairs[i][1], streams[0])
    torch.cuda.synchronize()
    pair_ms = sum(ev.elapsed_ms(i) for i in range(args.steps)) / args.steps
    gemm_ms = event_ms - pair_ms
    ev.close()
    st = moer.decode_load_stats(stats.cpu())[0]
    print(f"[bench] {ms_step * 1e3:.1f} us/step (wall {t_wall / args.steps * 1e6:.1f} us), "
          f"gate GEMM {gemm_ms * 1e3:.1f} us ({event_ms * 1e3:.1f} us between its events, "
          f"{pair_ms * 1e3:.1f} us for an empty pair); last imbalance "
          f"{st['imbalance']:.3f}", file=sys.stderr, flush=True)

    dc = None
    if not args.no_dispatch_combine:
        dc = time_dispatch_combine(moer, torch, wl, xs[0], outs, streams[0], args.steps)
        print(f"[bench] dispatch {dc['dispatch']['us']:.1f} us, combine "
              f"{dc['combine']['us']:.1f} us", file=sys.stderr, flush=True)

    fl = None
    if not args.no_forcible:
        fl = time_forcible_layout(moer, torch, wl, outs, streams[0], args.steps)
        print(f"[bench] layout (INDICES mode): routed ids {fl['routed_ids']['us']:.1f} us, "
              f"balanced ids {fl['balanced_ids']['us']:.1f} us", file=sys.stderr, flush=True)

    cp = time_capacity(moer, torch, wl, xs[0], Wd, bias, streams[0], args.steps)
    print(f"[bench] capacity {cp['capacity']}: {cp['dsv3_group']['us']:.1f} us "
          f"({cp['dsv3_group']['rerouted']} rerouted), with celebrity offsets "
          f"{cp['collapse_offsets']['us']:.1f} us ({cp['collapse_offsets']['rerouted']} rerouted, "
          f"{cp['collapse_offsets']['dropped']} dropped)", file=sys.stderr, flush=True)
    bs = time_balance_step(moer, torch, wl, outs, streams[0], args.steps)
    print(f"[bench] balance step: sign {bs['sign']['us']:.1f} us, proportional+EMA "
          f"{bs['proportional_ema_every4']['us']:.1f} us", file=sys.stderr, flush=True)

    esize = 2 if wl.dtype == workloads.BF16 else 4
    alg_bytes = L * (T + N) * wl.d * esize  # x + W_g of every layer per launch
    achieved = alg_bytes / (gemm_ms * 1e-3) / 1e9
    traffic = measured_traffic()
    line = {
        "metric": METRIC,
        "value": T * L / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
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
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": "gate_gemm", "kernel_us": gemm_ms * 1e3,
                     "event_pair_us": event_ms * 1e3, "empty_pair_us": pair_ms * 1e3,
                     "alg_bytes": alg_bytes},
    }
    if dc is not None:
        line["dispatch_combine"] = dc
    if fl is not None:
        line["forcible_layout"] = fl
    line["balance_step"] = bs
    line["capacity_route"] = cp
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on one batch", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(wl, {"x": xs_cpu[0], "W": W, "bias": b0})
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
