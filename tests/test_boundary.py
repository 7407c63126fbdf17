"""The C-ABI boundary on the CPU: the library loads, exports every function
include/moer.h declares, and its host-side validation returns the documented
status codes before anything reaches a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

import top_expert_routing_gate_amd as moer
from top_expert_routing_gate_amd import _moer

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moer.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return sorted(set(re.findall(r"\b(moer_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert set(names) == set(moer.EXPORTED), names
    lib = ctypes.CDLL(moer.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    nm = subprocess.run(["nm", "-D", "--defined-only", moer.LIB_PATH], capture_output=True,
                        text=True, check=True).stdout
    exported = set(re.findall(r"\bT (moer_\w+)", nm))
    assert set(names) <= exported


def test_abi_version_and_status_strings():
    assert moer.moer_abi_version() == 2
    assert _moer._status_name(moer.MOER_EINVAL) == "MOER_EINVAL"
    assert _moer._status_name(moer.MOER_EWORKSPACE) == "MOER_EWORKSPACE"


def _desc(**kw):
    base = dict(n_layers=1, T=16384, d=7168, N=256, K=8, n_groups=8, topk_groups=4, n_shared=0,
                score_fn=moer.MOER_SIGMOID, dtype=moer.MOER_BF16, input=moer.MOER_IN_HIDDEN)
    base.update(kw)
    return moer.make_desc(**base)


def _route_raw(desc, io=None, ws=None, ws_bytes=0):
    lib = _moer._lib
    io = io if io is not None else _moer.MoerRouteIO()
    st = lib.moer_route(ctypes.byref(desc) if desc is not None else None, ctypes.byref(io),
                        ws, ws_bytes, None)
    return st, lib.moer_last_error().decode()


@pytest.mark.parametrize("kw,frag", [
    (dict(n_layers=0), "n_layers"),
    (dict(T=-1), "T must"),
    (dict(N=0), "N must"),
    (dict(N=257, n_groups=1, topk_groups=1), "N must"),
    (dict(K=0), "K must"),
    (dict(K=300), "K must"),
    (dict(K=8, n_shared=9), "K + n_shared"),
    (dict(n_groups=7), "n_groups must divide"),
    (dict(topk_groups=9), "topk_groups"),
    (dict(N=8, n_groups=8, topk_groups=4, K=2), "at least 2 experts"),
    (dict(N=16, n_groups=8, topk_groups=1, K=3), "topk_groups * N/n_groups"),
    (dict(d=7170), "d % 8"),
    (dict(score_fn=5), "score_fn"),
    (dict(input=7), "input mode"),
    (dict(dtype=9), "dtype"),
    (dict(T=2**28, n_shared=8), "2^31"),
])
def test_invalid_descriptors_are_rejected(kw, frag):
    d = _desc(**kw)
    st, msg = _route_raw(d)
    assert st == moer.MOER_EINVAL and frag in msg, msg
    assert moer.moer_route_workspace_bytes(d) == 0


def test_null_descriptor_and_io():
    st, msg = _route_raw(None)
    assert st == moer.MOER_EINVAL and "desc" in msg
    d = _desc()
    st = _moer._lib.moer_route(ctypes.byref(d), None, None, 0, None)
    assert st == moer.MOER_EINVAL


@pytest.mark.parametrize("kw", [
    dict(n_groups=128, topk_groups=64),           # 128 groups of 2 among 256 experts
    dict(N=96, n_groups=8, topk_groups=4),         # groups of 12 (not a power of two)
    dict(N=255, n_groups=17, topk_groups=3),       # groups of 15
    dict(N=60, n_groups=20, topk_groups=3, K=6),   # groups of 3
])
def test_any_group_geometry_accepted(kw):
    # every group size >= 2 that divides N is valid for the method and has a
    # kernel: the descriptor passes, and the call stops at the empty io
    d = _desc(**kw)
    st, msg = _route_raw(d)
    assert st == moer.MOER_EINVAL and "x and w_gate" in msg, msg
    assert moer.moer_route_workspace_bytes(d) > 0


def test_missing_buffers_and_workspace():
    d = _desc()
    st, msg = _route_raw(d)
    assert st == moer.MOER_EINVAL and "x and w_gate" in msg
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
    io = _moer.MoerRouteIO(x=fake, w_gate=fake)
    st, msg = _route_raw(d, io)
    assert st == moer.MOER_EINVAL and "topk_idx" in msg
    io = _moer.MoerRouteIO(x=fake, w_gate=fake, topk_idx=fake, topk_w=fake)
    st, msg = _route_raw(d, io)
    assert st == moer.MOER_EINVAL and "counts" in msg
    # every optional output requested: the call needs the full advertised workspace
    io = _moer.MoerRouteIO(x=fake, w_gate=fake, topk_idx=fake, topk_w=fake, counts=fake,
                           offsets=fake, perm=fake, agg_entropy=fake)
    st, msg = _route_raw(d, io)
    assert st == moer.MOER_EWORKSPACE and "NULL" in msg
    need = moer.moer_route_workspace_bytes(d)
    st, msg = _route_raw(d, io, fake, need - 1)
    assert st == moer.MOER_EWORKSPACE and str(need) in msg
    io.ev_gemm_begin = fake
    st, msg = _route_raw(d, io, fake, need)
    assert st == moer.MOER_EINVAL and "ev_gemm" in msg
    io.ev_gemm_begin = None
    for u in (float("nan"), -1e-3, float("inf")):
        io.bias_update, io.bias_update_u = fake, u
        st, msg = _route_raw(d, io, fake, need)
        assert st == moer.MOER_EINVAL and "bias_update_u" in msg, u


def test_misaligned_inputs_are_rejected():
    d = _desc()
    ok, odd = ctypes.c_void_p(0x1000), ctypes.c_void_p(0x1008)  # never dereferenced
    need = moer.moer_route_workspace_bytes(d)
    full = dict(topk_idx=ok, topk_w=ok, counts=ok, offsets=ok, perm=ok)
    for field in ("x", "w_gate"):
        io = _moer.MoerRouteIO(**{**full, "x": ok, "w_gate": ok, field: odd})
        st, msg = _route_raw(d, io, ok, need)
        assert st == moer.MOER_EINVAL and "16-byte" in msg, (field, msg)
    for field in ("bias", "logit_offset"):
        io = _moer.MoerRouteIO(**{**full, "x": ok, "w_gate": ok, field: odd})
        st, msg = _route_raw(d, io, ok, need)
        assert st == moer.MOER_EINVAL and "16-byte" in msg, (field, msg)
    ds = _desc(input=moer.MOER_IN_SCORES, d=0)
    io = _moer.MoerRouteIO(**{**full, "scores": odd})
    st, msg = _route_raw(ds, io, ok, moer.moer_route_workspace_bytes(ds))
    assert st == moer.MOER_EINVAL and "16-byte" in msg, msg


def test_binding_refuses_buffers_of_the_wrong_size():
    # shapes are checked before anything reaches the library (CPU tensors
    # would be refused later anyway; the size check comes first)
    import torch

    x = torch.zeros(2, 8, 64, dtype=torch.bfloat16)
    w = torch.zeros(2, 256, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="bias"):
        moer.route(x, w, K=8, bias=torch.zeros(256))          # one layer's bias for two layers
    with pytest.raises(ValueError, match="w_gate"):
        moer.route(x, torch.zeros(2, 256, 32, dtype=torch.bfloat16), K=8)   # d differs
    with pytest.raises(ValueError, match="w_gate"):
        moer.route(x, torch.zeros(1, 256, 64, dtype=torch.bfloat16), K=8)   # L differs
    with pytest.raises(ValueError, match="logit_offset"):
        moer.route(x, w, K=8, logit_offset=torch.zeros(128))
    with pytest.raises(ValueError, match="bias_update"):
        moer.route(x, w, K=8, bias_update=torch.zeros(2, 128))
    with pytest.raises(ValueError, match="idx_in"):
        moer.route(idx_in=torch.zeros(1, 8, 3, dtype=torch.int32), K=8, N=256)
    # the marshalling layer checks every buffer against the descriptor
    desc = moer.make_desc(n_layers=2, T=8, d=64, N=256, K=8)
    with pytest.raises(ValueError, match="counts"):
        _moer._route_io(desc, counts=torch.zeros(256, dtype=torch.int32))


def test_noalloc_rejects_routers_beyond_its_scratch_before_any_gpu_call():
    # validation and the size check come before the device is touched
    d = _desc(capacity=640)
    assert moer.moer_route_workspace_bytes(d) > moer.MOER_NOALLOC_SCRATCH_BYTES
    st = _moer._lib.moer_route_noalloc(ctypes.byref(d), ctypes.byref(_moer.MoerRouteIO()), None)
    msg = _moer._lib.moer_last_error().decode()
    assert st == moer.MOER_EWORKSPACE and "static scratch" in msg, msg
    st = _moer._lib.moer_route_noalloc(ctypes.byref(_desc(n_layers=0)),
                                       ctypes.byref(_moer.MoerRouteIO()), None)
    assert st == moer.MOER_EINVAL
    # the five workloads without a capacity fit
    assert moer.moer_route_workspace_bytes(_desc()) <= moer.MOER_NOALLOC_SCRATCH_BYTES


def test_workspace_sizes():
    # dsv3 shape: partial affinities (one or more depth ranges of 16 MiB each)
    # + entropy partials + block histograms
    n = moer.moer_route_workspace_bytes(_desc())
    assert 16384 * 256 * 4 < n < 5 * 16384 * 256 * 4
    n_scores = moer.moer_route_workspace_bytes(_desc(input=moer.MOER_IN_SCORES))
    assert n_scores < 2 * 2**20
    n_idx = moer.moer_route_workspace_bytes(_desc(input=moer.MOER_IN_INDICES))
    assert 0 < n_idx < n_scores
    assert moer.moer_route_workspace_bytes(_desc(T=0)) > 0


def test_stats_and_bias_validation():
    lib = _moer._lib
    fake = ctypes.c_void_p(0x1000)
    assert lib.moer_load_stats(None, 1, 4, 4, fake, None) == moer.MOER_EINVAL
    assert lib.moer_load_stats(fake, 0, 4, 4, fake, None) == moer.MOER_EINVAL
    assert lib.moer_load_stats(fake, 1, 4, 3, fake, None) == moer.MOER_EINVAL
    assert lib.moer_bias_update(fake, None, 1, 4, 4, ctypes.c_float(1e-3), None) == moer.MOER_EINVAL
    assert lib.moer_bias_update(fake, fake, 1, 4, 4, ctypes.c_float(float("nan")), None) == \
        moer.MOER_EINVAL
    assert lib.moer_bias_update(fake, fake, 1, 4, 4, ctypes.c_float(-1.0), None) == \
        moer.MOER_EINVAL


def _dispatch_raw(x=0x1000, row_bytes=14336, L=1, T=4, Kt=8, inv=0x2000, out=0x3000):
    st = _moer._lib.moer_dispatch(x, row_bytes, L, T, Kt, inv, out, None)
    return st, _moer._lib.moer_last_error().decode()


def _combine_raw(eo=0x1000, eo_dt=moer.MOER_BF16, w=0x2000, inv=0x3000, L=1, T=4, Kt=8, d=7168,
                 y=0x4000, y_dt=moer.MOER_BF16):
    st = _moer._lib.moer_combine(eo, eo_dt, w, inv, L, T, Kt, d, y, y_dt, None)
    return st, _moer._lib.moer_last_error().decode()


@pytest.mark.parametrize("kw,frag", [
    (dict(L=0), "n_layers"),
    (dict(T=-1), "T >= 0"),
    (dict(Kt=0), "Kt must"),
    (dict(Kt=17), "Kt must"),
    (dict(T=2**28, Kt=8), "2^31"),
    (dict(row_bytes=0), "row_bytes"),
    (dict(row_bytes=14344), "row_bytes"),
    (dict(x=None), "required"),
    (dict(inv=None), "required"),
    (dict(out=None), "required"),
    (dict(x=0x1008), "aligned"),
    (dict(out=0x3004), "aligned"),
])
def test_dispatch_rejects_bad_arguments(kw, frag):
    st, msg = _dispatch_raw(**kw)
    assert st == moer.MOER_EINVAL and frag in msg, msg


@pytest.mark.parametrize("kw,frag", [
    (dict(L=0), "n_layers"),
    (dict(Kt=0), "Kt must"),
    (dict(Kt=17), "Kt must"),
    (dict(d=0), "multiple of 8"),
    (dict(d=7164), "multiple of 8"),
    (dict(eo_dt=7), "MOER_BF16 or MOER_F32"),
    (dict(y_dt=-1), "MOER_BF16 or MOER_F32"),
    (dict(eo=None), "required"),
    (dict(w=None), "required"),
    (dict(inv=None), "required"),
    (dict(y=None), "required"),
    (dict(eo=0x1002), "aligned"),
    (dict(y=0x4008), "aligned"),
])
def test_combine_rejects_bad_arguments(kw, frag):
    st, msg = _combine_raw(**kw)
    assert st == moer.MOER_EINVAL and frag in msg, msg


def test_dispatch_and_combine_of_no_tokens_launch_nothing():
    # T = 0 returns before any device call, so it runs without a GPU
    assert _dispatch_raw(T=0, x=None, inv=None, out=None)[0] == moer.MOER_OK
    assert _combine_raw(T=0, eo=None, w=None, inv=None, y=None)[0] == moer.MOER_OK


@pytest.mark.parametrize("kw,frag", [
    (dict(N=0), "N must"),
    (dict(N=257), "N must"),
    (dict(K=0), "K must"),
    (dict(K=9, N=8), "K must"),
    (dict(ns=-1), "n_shared"),
    (dict(K=8, ns=9), "Kt must"),
    (dict(L=0), "n_layers"),
    (dict(T=2**28), "2^31"),
    (dict(idx=None), "required"),
])
def test_balanced_indices_reject_bad_arguments(kw, frag):
    a = dict(idx=0x1000, L=1, T=16, K=8, N=256, ns=0, first=0)
    a.update(kw)
    st = _moer._lib.moer_balanced_indices(a["idx"], a["L"], a["T"], a["K"], a["N"], a["ns"],
                                          a["first"], None)
    msg = _moer._lib.moer_last_error().decode()
    assert st == moer.MOER_EINVAL and frag in msg, msg


@pytest.mark.parametrize("kw,frag", [
    (dict(hot=None), "required"),
    (dict(counts=None), "required"),
    (dict(L=0), "n_layers"),
    (dict(stride=3, N=4), "stride >= N"),
])
def test_hotspot_accumulate_rejects_bad_arguments(kw, frag):
    a = dict(hot=0x1000, counts=0x2000, L=1, N=4, stride=4)
    a.update(kw)
    st = _moer._lib.moer_hotspot_accumulate(a["hot"], a["counts"], a["L"], a["N"], a["stride"],
                                            None)
    msg = _moer._lib.moer_last_error().decode()
    assert st == moer.MOER_EINVAL and frag in msg, msg


@pytest.mark.parametrize("kw,frag", [
    (dict(bias_mode=5), "bias_mode"),
    (dict(bias_mode=moer.MOER_BIAS_LOGIT, input=moer.MOER_IN_SCORES), "HIDDEN"),
    (dict(bias_mode=moer.MOER_BIAS_LOGIT, input=moer.MOER_IN_INDICES), "HIDDEN"),
])
def test_bias_mode_validation(kw, frag):
    d = _desc(**kw)
    st, msg = _route_raw(d)
    assert st == moer.MOER_EINVAL and frag in msg, msg


@pytest.mark.parametrize("kw,frag", [
    (dict(bias=None), "required"),
    (dict(counts=None), "required"),
    (dict(cfg=None), "required"),
    (dict(N=300), "N <= 256"),
    (dict(stride=100), "stride >= N"),
    (dict(rule=3), "unknown rule"),
    (dict(step=-1.0), "step must"),
    (dict(step=float("inf")), "step must"),
    (dict(step=float("nan")), "step must"),
    (dict(alpha=0.0), "alpha must"),
    (dict(alpha=1.5), "alpha must"),
    (dict(every=0), "every must"),
    (dict(alpha=0.5, loads=None), "loads state"),
    (dict(every=4, calls=None), "calls state"),
])
def test_balance_step_rejects_bad_arguments(kw, frag):
    a = dict(bias=0x1000, counts=0x2000, L=2, N=256, stride=256, rule=0, step=1e-3, alpha=1.0,
             every=1, loads=0x3000, calls=0x4000, cfg=True)
    a.update(kw)
    cfg = _moer.MoerBalanceCfg(a["rule"], a["step"], a["alpha"], a["every"])
    st = _moer._lib.moer_balance_step(a["bias"], a["counts"], a["L"], a["N"], a["stride"],
                                      ctypes.byref(cfg) if a["cfg"] else None, a["loads"],
                                      a["calls"], None)
    msg = _moer._lib.moer_last_error().decode()
    assert st == moer.MOER_EINVAL and frag in msg, msg


def test_balance_monitor_thresholds_and_streaks():
    # the statistics records here are hand-computed (the device writes them
    # in use); the monitor only applies the thresholds and keeps the streaks
    mon = moer.BalanceMonitor(8, cv_limit=0.2, hot_margin=0.5, persist=2)
    balanced = [64] * 8
    st_bal = {"total": 512, "mean": 64.0, "cv": 0.0}
    hot = [200, 40, 40, 40, 40, 56, 48, 48]           # expert 0 at 3.1x the mean
    # mean 64; deviations 136, -24 x4, -8, -16 x2: var = (18496 + 2304 + 64 + 512)/8
    cv = (21376 / 8) ** 0.5 / 64
    st_hot = {"total": 512, "mean": 64.0, "cv": cv}
    assert mon.observe(st_bal, balanced) == []
    assert mon.observe(st_hot, hot) == [("spread", cv)]        # one batch: no streak yet
    a2 = mon.observe(st_hot, hot)
    assert ("spread", cv) in a2 and ("hot", 0, 2) in a2
    assert all(a[0] != "hot" or a[1] == 0 for a in a2)          # 56 < 1.5 * 64 = 96
    assert mon.observe(st_bal, balanced) == [] and mon.streak[0] == 0
    # the spread limit sits exactly at the pages' 20 %: std/mean = sqrt(200)/100
    c = [120, 80, 100, 100]
    assert moer.BalanceMonitor(4).observe({"total": 400, "mean": 100.0, "cv": 0.1414}, c) == []
    # an empty batch resets the streaks
    mon.observe(st_hot, hot)
    assert mon.observe({"total": 0, "mean": 0.0, "cv": 0.0}, [0] * 8) == []
    assert mon.streak == [0] * 8


def test_capacity_validation():
    st, msg = _route_raw(_desc(capacity=-1))
    assert st == moer.MOER_EINVAL and "capacity" in msg, msg
    st, msg = _route_raw(_desc(capacity=640, input=moer.MOER_IN_INDICES))
    assert st == moer.MOER_EINVAL and "capacity" in msg, msg
    # the capacity rounds need their own workspace
    assert (moer.moer_route_workspace_bytes(_desc(capacity=640)) >
            moer.moer_route_workspace_bytes(_desc()) + 16384 * 256 * 8)


def test_expert_capacity_is_the_pages_formula():
    # dailyaiworld, production testing: capacity = 1.25 x (batch x top_k /
    # experts), rounded up; values worked by hand
    assert moer.expert_capacity(16384, 8, 256) == 640
    assert moer.expert_capacity(64, 1, 4) == 20
    assert moer.expert_capacity(100, 3, 7) == 54      # 1.25 * 300 / 7 = 53.57...
    assert moer.expert_capacity(4096, 2, 8) == 1280
    assert moer.expert_capacity(128, 8, 256) == 5     # 1.25 * 4 = 5 exactly: not rounded up
    assert moer.expert_capacity(100, 3, 7, factor="1") == 43  # 42.86... rounded up
