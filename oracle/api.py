"""ctypes marshalling for the C oracle (moero.c). Test infrastructure only.

No arithmetic of the method is done here: every step calls into moero.c,
except ``route``, which only chains those calls in the order the pages give
(affinities -> [logit bias] -> scores -> selection -> layout -> entropy).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moero.c")
_LIB = os.path.join(_HERE, "libmoero.so")
# a prebuilt oracle library to load instead (the pin tests' mutation check
# points this at deliberately broken builds)
_LIB_OVERRIDE = os.environ.get("MOERO_LIB")

SOFTMAX, SIGMOID = 0, 1


def build_oracle():
    """Compile moero.c with gcc (no FMA contraction, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-o", _LIB, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    return _LIB


class _Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("T", "N", "K", "n_groups", "topk_groups", "n_shared")]


class _Stats(ctypes.Structure):
    _fields_ = [("total", ctypes.c_int64), ("max_load", ctypes.c_int64),
                ("argmax", ctypes.c_int64), ("capacity", ctypes.c_int64),
                ("mean", ctypes.c_double), ("imbalance", ctypes.c_double),
                ("h_load_bits", ctypes.c_double), ("cv", ctypes.c_double)]


_lib = None


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build_oracle()
            lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32 = ctypes.c_int32
        lib.moero_affinities.argtypes = [P, P, P, i32, i32, i32, P]
        lib.moero_scores.argtypes = [P, i32, i32, i32, P]
        lib.moero_select.argtypes = [ctypes.POINTER(_Cfg), P, P, P, P, P, P, P]
        lib.moero_select.restype = ctypes.c_int
        lib.moero_capacity_route.argtypes = [ctypes.POINTER(_Cfg), P, P, P, i32, P, P, P, P]
        lib.moero_capacity_route.restype = ctypes.c_int
        lib.moero_agg_entropy.argtypes = [P, i32, i32]
        lib.moero_agg_entropy.restype = ctypes.c_double
        lib.moero_layout.argtypes = [P, i32, i32, i32, P, P, P, P]
        lib.moero_load_stats.argtypes = [P, i32, ctypes.POINTER(_Stats)]
        lib.moero_bias_update.argtypes = [P, P, i32, ctypes.c_float]
        lib.moero_dispatch.argtypes = [P, ctypes.c_int64, i32, i32, P, P]
        lib.moero_combine.argtypes = [P, P, P, i32, i32, i32, P]
        lib.moero_balanced_indices.argtypes = [i32, i32, i32, i32, i32, P]
        lib.moero_hotspot_accumulate.argtypes = [P, P, i32, i32, i32]
        lib.moero_logit_bias.argtypes = [P, P, i32, i32]
        lib.moero_balance_step.argtypes = [P, P, i32, i32, ctypes.c_float, ctypes.c_float, i32,
                                           P, P]
        lib.moero_num_threads.restype = ctypes.c_int
        lib.moero_set_num_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dt):
    return None if a is None else np.ascontiguousarray(a, dtype=dt)


def num_threads():
    return int(_load().moero_num_threads())


def set_num_threads(n):
    _load().moero_set_num_threads(int(n))


def affinities(x, W, offset=None):
    """h[t,e] = sum_k x[t,k] W[e,k] (+ offset[e]) in fp64. x [T,d], W [N,d]."""
    x = _c(x, np.float32); W = _c(W, np.float32); offset = _c(offset, np.float32)
    T, d = x.shape
    N = W.shape[0]
    assert W.shape[1] == d
    h = np.empty((T, N), np.float64)
    _load().moero_affinities(_p(x), _p(W), _p(offset), T, d, N, _p(h))
    return h


def scores(h, score_fn):
    h = _c(h, np.float64)
    T, N = h.shape
    s = np.empty_like(h)
    _load().moero_scores(_p(h), T, N, int(score_fn), _p(s))
    return s


def select(s32, s64, bias, K, n_groups=1, topk_groups=1, n_shared=0):
    """Routing decision per token. Returns idx [T,Kt] int32, w [T,Kt] f32,
    tok_H [T] f64 (bits) and gap [T] f64."""
    s32 = _c(s32, np.float32); s64 = _c(s64, np.float64); bias = _c(bias, np.float32)
    T, N = s32.shape
    Kt = K + n_shared
    cfg = _Cfg(T, N, K, n_groups, topk_groups, n_shared)
    idx = np.empty((T, Kt), np.int32)
    w = np.empty((T, Kt), np.float32)
    H = np.empty(T, np.float64)
    gap = np.empty(T, np.float64)
    rc = _load().moero_select(ctypes.byref(cfg), _p(s32), _p(s64), _p(bias),
                              _p(idx), _p(w), _p(H), _p(gap))
    if rc != 0:
        raise ValueError("oracle: invalid routing configuration")
    return idx, w, H, gap


def capacity_route(s32, s64, bias, K, cap, n_groups=1, topk_groups=1, n_shared=0):
    """Capacity-limited routing. Returns idx [T,Kt] int32 (-1 = dropped),
    w [T,Kt] f32, and the numbers of rerouted and dropped slots."""
    s32 = _c(s32, np.float32); s64 = _c(s64, np.float64); bias = _c(bias, np.float32)
    T, N = s32.shape
    Kt = K + n_shared
    cfg = _Cfg(T, N, K, n_groups, topk_groups, n_shared)
    idx = np.empty((T, Kt), np.int32)
    w = np.empty((T, Kt), np.float32)
    rr, dr = ctypes.c_int64(), ctypes.c_int64()
    rc = _load().moero_capacity_route(ctypes.byref(cfg), _p(s32), _p(s64), _p(bias), int(cap),
                                      _p(idx), _p(w), ctypes.byref(rr), ctypes.byref(dr))
    if rc != 0:
        raise ValueError("oracle: invalid routing configuration")
    return idx, w, rr.value, dr.value


def agg_entropy(s64):
    s64 = _c(s64, np.float64)
    T, N = s64.shape
    return float(_load().moero_agg_entropy(_p(s64), T, N))


def layout(idx, Nb):
    """counts [Nb], offsets [Nb+1], perm [T*Kt], inv_perm [T*Kt] (int32)."""
    idx = _c(idx, np.int32)
    T, Kt = idx.shape
    counts = np.empty(Nb, np.int32)
    offsets = np.empty(Nb + 1, np.int32)
    perm = np.empty(T * Kt, np.int32)
    inv = np.empty(T * Kt, np.int32)
    _load().moero_layout(_p(idx), T, Kt, Nb, _p(counts), _p(offsets), _p(perm), _p(inv))
    return counts, offsets, perm, inv


def dispatch(x, perm, Kt, out=None):
    """Rows of x [T, d] (any dtype, copied as bytes) gathered into layout
    order: returns [T*Kt, d]; rows whose perm entry is -1 keep ``out``'s
    contents (zeros when ``out`` is None)."""
    x = np.ascontiguousarray(x)
    perm = _c(perm, np.int32)
    T = x.shape[0]
    assert perm.shape == (T * Kt,)
    if out is None:
        out = np.zeros((T * Kt,) + x.shape[1:], x.dtype)
    else:
        out = np.array(out, dtype=x.dtype, copy=True, order="C")
        assert out.shape == (T * Kt,) + x.shape[1:]
    row_bytes = x.dtype.itemsize * int(np.prod(x.shape[1:], dtype=np.int64))
    _load().moero_dispatch(_p(x), row_bytes, T, Kt, _p(perm), _p(out))
    return out


def combine(out_rows, w, perm):
    """y [T, d] fp64 = per token, the w-weighted sum of its slots' rows of
    out_rows [T*Kt, d] (given as exact values; converted to fp64 here)."""
    w = _c(w, np.float32)
    T, Kt = w.shape
    out_rows = _c(out_rows, np.float64)
    d = out_rows.shape[1]
    assert out_rows.shape == (T * Kt, d)
    perm = _c(perm, np.int32)
    y = np.empty((T, d), np.float64)
    _load().moero_combine(_p(out_rows), _p(w), _p(perm), T, Kt, d, _p(y))
    return y


def balanced_indices(T, K, N, n_shared=0, first=0):
    """Forcible-balance expert ids [T, K + n_shared] int32."""
    idx = np.empty((T, K + n_shared), np.int32)
    _load().moero_balanced_indices(T, K, N, n_shared, int(first), _p(idx))
    return idx


def hotspot_accumulate(hot, counts, N):
    """Returns hot [L, N] int64 plus counts[:, :N] (inputs are not modified)."""
    hot = np.array(hot, dtype=np.int64, copy=True, order="C")
    counts = _c(np.atleast_2d(counts), np.int32)
    L, stride = counts.shape
    assert hot.shape == (L, N)
    _load().moero_hotspot_accumulate(_p(hot), _p(counts), L, N, stride)
    return hot


def logit_bias(h, b):
    """Returns h [T,N] fp64 with the fp32 bias b [N] added to every row."""
    h = np.array(h, dtype=np.float64, copy=True, order="C")
    b = _c(b, np.float32)
    T, N = h.shape
    _load().moero_logit_bias(_p(h), _p(b), T, N)
    return h


SIGN, PROPORTIONAL = 0, 1


def balance_step(bias, counts, *, rule=SIGN, step=1e-3, alpha=1.0, every=1, loads=None,
                 calls=None):
    """One balancing step; returns (bias, loads, calls) updated copies."""
    b = np.array(bias, dtype=np.float32, copy=True)
    counts = _c(counts, np.int32)
    N = counts.shape[0]
    ld = None if loads is None else np.array(loads, dtype=np.float32, copy=True)
    cl = None if calls is None else np.array([calls], dtype=np.int32)
    _load().moero_balance_step(_p(b), _p(counts), N, int(rule), ctypes.c_float(step),
                               ctypes.c_float(alpha), int(every), _p(ld), _p(cl))
    return b, ld, None if cl is None else int(cl[0])


def load_stats(counts):
    counts = _c(counts, np.int32)
    st = _Stats()
    _load().moero_load_stats(_p(counts), counts.shape[0], ctypes.byref(st))
    return {n: getattr(st, n) for n, _ in _Stats._fields_}


def bias_update(bias, counts, u=1e-3):
    """Returns the updated fp32 bias (the input array is not modified)."""
    b = np.array(bias, dtype=np.float32, copy=True)
    counts = _c(counts, np.int32)
    _load().moero_bias_update(_p(b), _p(counts), counts.shape[0], ctypes.c_float(u))
    return b


def route(*, K, score_fn, x=None, W=None, offset=None, s32=None, idx_in=None, bias=None,
          n_groups=1, topk_groups=1, n_shared=0, N=None, bias_mode="score"):
    """One router layer through the oracle, in the order of the pages.

    Input is one of: hidden states (x [T,d], W [N,d], fp32 holding the exact
    input values), fp32 scores s32 [T,N], or supplied indices idx_in [T,Kt].
    bias_mode "score" adds the bias to the scores for the selection only;
    "logit" (hidden states only) adds it to the logits.
    """
    if bias_mode == "logit" and (x is None or idx_in is not None or s32 is not None):
        raise ValueError("logit-space bias needs hidden-state input")
    out = {}
    if idx_in is None:
        if s32 is None:
            h = affinities(x, W, offset)
            if bias_mode == "logit":
                h = logit_bias(h, bias)
                bias = None
            s64 = scores(h, score_fn)
            s32 = s64.astype(np.float32)
            out["h"] = h
        else:
            s32 = np.ascontiguousarray(s32, np.float32)
            s64 = s32.astype(np.float64)
        N = s32.shape[1]
        idx, w, H, gap = select(s32, s64, bias, K, n_groups, topk_groups, n_shared)
        out.update(s32=s32, s64=s64, idx=idx, w=w, tok_H=H, gap=gap,
                   agg_H=agg_entropy(s64))
    else:
        idx = np.ascontiguousarray(idx_in, np.int32)
        out["idx"] = idx
    Nb = N + n_shared
    counts, offsets, perm, inv = layout(idx, Nb)
    out.update(counts=counts, offsets=offsets, perm=perm, inv_perm=inv)
    return out
