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
    assert moer.moer_abi_version() == 1
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


def test_unsupported_group_geometry():
    # 128 groups of 2 among 256 experts: valid for the method, not for these kernels
    d = _desc(n_groups=128, topk_groups=64)
    st, msg = _route_raw(d)
    assert st == moer.MOER_EUNSUPPORTED and "group size" in msg
    d = _desc(N=96, n_groups=8, topk_groups=4)  # groups of 12 (not a power of two)
    assert _route_raw(d)[0] == moer.MOER_EUNSUPPORTED


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
