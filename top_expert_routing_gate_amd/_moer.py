"""ctypes binding of libmoer.so — argument marshalling only.

The names match the C ABI in include/moer.h (moer_route, moer_load_stats,
moer_bias_update, ...). Torch supplies device memory and the current stream;
every step of the router runs in the library's HIP kernels. There is no
fallback: if the library is not built, importing this module raises.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoer.so")

MOER_OK, MOER_EINVAL, MOER_EUNSUPPORTED, MOER_EWORKSPACE, MOER_EHIP = range(5)
MOER_SOFTMAX, MOER_SIGMOID = 0, 1
MOER_BF16, MOER_F32 = 0, 1
MOER_IN_HIDDEN, MOER_IN_SCORES, MOER_IN_INDICES = 0, 1, 2
MOER_BIAS_SCORE, MOER_BIAS_LOGIT = 0, 1
MOER_RULE_SIGN, MOER_RULE_PROPORTIONAL = 0, 1
MOER_MAX_EXPERTS, MOER_MAX_SLOTS = 256, 16

EXPORTED = ("moer_route_workspace_bytes", "moer_route", "moer_route_noalloc", "moer_load_stats",
            "moer_bias_update",
            "moer_balance_step", "moer_dispatch", "moer_combine", "moer_balanced_indices",
            "moer_hotspot_accumulate",
            "moer_status_str", "moer_last_error", "moer_abi_version")


class MoerRouteDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("n_layers", "T", "d", "N", "K", "n_groups", "topk_groups", "n_shared",
                 "score_fn", "dtype", "input", "bias_mode", "capacity")]


class MoerBalanceCfg(ctypes.Structure):
    _fields_ = [("rule", ctypes.c_int32), ("step", ctypes.c_float), ("alpha", ctypes.c_float),
                ("every", ctypes.c_int32)]


class MoerRouteIO(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("x", "w_gate", "scores", "idx_in", "bias", "logit_offset", "h_out", "topk_w",
                 "tok_entropy", "agg_entropy", "topk_idx", "counts", "offsets", "perm",
                 "inv_perm", "ev_gemm_begin", "ev_gemm_end", "load_stats", "bias_update")] + \
        [("bias_update_u", ctypes.c_float), ("cap_stats", ctypes.c_void_p),
         ("ev_select_wait", ctypes.c_void_p)]


class MoerLoadStats(ctypes.Structure):
    _fields_ = [("total", ctypes.c_int64), ("max_load", ctypes.c_int64),
                ("argmax", ctypes.c_int64), ("capacity", ctypes.c_int64),
                ("mean", ctypes.c_double), ("imbalance", ctypes.c_double),
                ("h_load_bits", ctypes.c_double), ("cv", ctypes.c_double)]


LOAD_STATS_FIELDS = [n for n, _ in MoerLoadStats._fields_]
assert ctypes.sizeof(MoerLoadStats) == 64


class MoerError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "(or python top_expert_routing_gate_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32 = ctypes.c_int32
    lib.moer_route_workspace_bytes.argtypes = [ctypes.POINTER(MoerRouteDesc)]
    lib.moer_route_workspace_bytes.restype = ctypes.c_size_t
    lib.moer_route.argtypes = [ctypes.POINTER(MoerRouteDesc), ctypes.POINTER(MoerRouteIO), P,
                               ctypes.c_size_t, P]
    lib.moer_route.restype = ctypes.c_int
    lib.moer_route_noalloc.argtypes = [ctypes.POINTER(MoerRouteDesc), ctypes.POINTER(MoerRouteIO), P]
    lib.moer_route_noalloc.restype = ctypes.c_int
    lib.moer_load_stats.argtypes = [P, i32, i32, i32, P, P]
    lib.moer_load_stats.restype = ctypes.c_int
    lib.moer_bias_update.argtypes = [P, P, i32, i32, i32, ctypes.c_float, P]
    lib.moer_bias_update.restype = ctypes.c_int
    lib.moer_dispatch.argtypes = [P, ctypes.c_int64, i32, i32, i32, P, P, P]
    lib.moer_dispatch.restype = ctypes.c_int
    lib.moer_combine.argtypes = [P, ctypes.c_int, P, P, i32, i32, i32, i32, P, ctypes.c_int, P]
    lib.moer_combine.restype = ctypes.c_int
    lib.moer_balance_step.argtypes = [P, P, i32, i32, i32, ctypes.POINTER(MoerBalanceCfg), P, P, P]
    lib.moer_balance_step.restype = ctypes.c_int
    lib.moer_balanced_indices.argtypes = [P, i32, i32, i32, i32, i32, i32, P]
    lib.moer_balanced_indices.restype = ctypes.c_int
    lib.moer_hotspot_accumulate.argtypes = [P, P, i32, i32, i32, P]
    lib.moer_hotspot_accumulate.restype = ctypes.c_int
    lib.moer_status_str.argtypes = [ctypes.c_int]
    lib.moer_status_str.restype = ctypes.c_char_p
    lib.moer_last_error.restype = ctypes.c_char_p
    lib.moer_abi_version.restype = ctypes.c_int
    return lib


_lib = _load()


def _status_name(st):
    return _lib.moer_status_str(st).decode()


def _check(st):
    if st != MOER_OK:
        raise MoerError(st, _lib.moer_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError("router buffers must be device tensors")
    if not t.is_contiguous():
        raise ValueError("router buffers must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def moer_abi_version():
    return int(_lib.moer_abi_version())


def make_desc(*, T, N, K, n_layers=1, d=0, n_groups=1, topk_groups=1, n_shared=0,
              score_fn=MOER_SIGMOID, dtype=MOER_BF16, input=MOER_IN_HIDDEN,
              bias_mode=MOER_BIAS_SCORE, capacity=0):
    return MoerRouteDesc(n_layers, T, d, N, K, n_groups, topk_groups, n_shared, score_fn, dtype,
                         input, bias_mode, capacity)


def moer_route_workspace_bytes(desc):
    return int(_lib.moer_route_workspace_bytes(ctypes.byref(desc)))


def _route_io(desc, *, x=None, w_gate=None, scores=None, idx_in=None, bias=None,
              logit_offset=None, h_out=None, topk_w=None, tok_entropy=None, agg_entropy=None,
              topk_idx=None, counts=None, offsets=None, perm=None, inv_perm=None,
              ev_gemm_begin=None, ev_gemm_end=None, load_stats=None, bias_update=None,
              bias_update_u=0.0, cap_stats=None, ev_select_wait=None):
    for name, t, dt in (("x", x, None), ("w_gate", w_gate, None), ("scores", scores, torch.float32),
                        ("idx_in", idx_in, torch.int32), ("bias", bias, torch.float32),
                        ("logit_offset", logit_offset, torch.float32),
                        ("h_out", h_out, torch.float32), ("topk_w", topk_w, torch.float32),
                        ("tok_entropy", tok_entropy, torch.float32),
                        ("agg_entropy", agg_entropy, torch.float32),
                        ("topk_idx", topk_idx, torch.int32), ("counts", counts, torch.int32),
                        ("offsets", offsets, torch.int32), ("perm", perm, torch.int32),
                        ("inv_perm", inv_perm, torch.int32), ("cap_stats", cap_stats, torch.int32),
                        ("bias_update", bias_update, torch.float32)):
        if t is not None and dt is not None and t.dtype != dt:
            raise TypeError(f"{name} must be {dt}, got {t.dtype}")
    if x is not None:
        want = torch.bfloat16 if desc.dtype == MOER_BF16 else torch.float32
        if x.dtype != want or (w_gate is not None and w_gate.dtype != want):
            raise TypeError(f"x and w_gate must be {want}")
    # element counts the kernels index (include/moer.h): a buffer of another
    # size would be read or written out of bounds, so it is refused here
    L, T, d, N = desc.n_layers, desc.T, desc.d, desc.N
    Kt, Nb = desc.K + desc.n_shared, desc.N + desc.n_shared
    for name, t, n in (("x", x, L * T * d), ("w_gate", w_gate, L * N * d),
                       ("scores", scores, L * T * N), ("idx_in", idx_in, L * T * Kt),
                       ("bias", bias, L * N), ("logit_offset", logit_offset, N),
                       ("h_out", h_out, L * T * N), ("topk_w", topk_w, L * T * Kt),
                       ("tok_entropy", tok_entropy, L * T), ("agg_entropy", agg_entropy, L),
                       ("topk_idx", topk_idx, L * T * Kt), ("counts", counts, L * Nb),
                       ("offsets", offsets, L * (Nb + 1)), ("perm", perm, L * T * Kt),
                       ("inv_perm", inv_perm, L * T * Kt), ("cap_stats", cap_stats, L * 2),
                       ("bias_update", bias_update, L * N)):
        if t is not None and t.numel() != n:
            raise ValueError(f"{name} has {t.numel()} elements; this router needs {n} "
                             f"(L={L}, T={T}, d={d}, N={N}, Kt={Kt})")
    if load_stats is not None and load_stats.numel() * load_stats.element_size() < 64 * desc.n_layers:
        raise ValueError("load_stats needs 64 bytes per layer")
    return MoerRouteIO(_ptr(x), _ptr(w_gate), _ptr(scores), _ptr(idx_in), _ptr(bias),
                       _ptr(logit_offset), _ptr(h_out), _ptr(topk_w), _ptr(tok_entropy),
                       _ptr(agg_entropy), _ptr(topk_idx), _ptr(counts), _ptr(offsets), _ptr(perm),
                       _ptr(inv_perm), ev_gemm_begin, ev_gemm_end, _ptr(load_stats),
                       _ptr(bias_update), float(bias_update_u), _ptr(cap_stats), ev_select_wait)


def moer_route(desc, *, workspace, stream=None, **buffers):
    """Calls moer_route on device tensors (shapes and dtypes as in moer.h)."""
    io = _route_io(desc, **buffers)
    ws = workspace
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.moer_route(ctypes.byref(desc), ctypes.byref(io), _ptr(ws), nbytes,
                           _stream(stream)))


MOER_NOALLOC_SCRATCH_BYTES = 40 << 20


def moer_route_noalloc(desc, *, stream=None, **buffers):
    """Calls moer_route_noalloc (the library's static scratch instead of a
    workspace) on device tensors."""
    io = _route_io(desc, **buffers)
    _check(_lib.moer_route_noalloc(ctypes.byref(desc), ctypes.byref(io), _stream(stream)))


class PreparedRoute:
    """One moer_route call whose arguments are marshalled once, for loops that
    route into the same buffers again and again (the tensors must stay alive
    and in place). Calling it enqueues moer_route with those arguments; only
    the two profiling events may change per call."""

    def __init__(self, desc, *, workspace, stream=None, **buffers):
        self.desc = desc
        self.io = _route_io(desc, **buffers)
        self._keep = (workspace, buffers)
        nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        self._args = (ctypes.byref(self.desc), ctypes.byref(self.io), _ptr(workspace), nbytes,
                      _stream(stream))

    def __call__(self, ev_gemm_begin=None, ev_gemm_end=None, ev_select_wait=None):
        self.io.ev_gemm_begin = ev_gemm_begin
        self.io.ev_gemm_end = ev_gemm_end
        self.io.ev_select_wait = ev_select_wait
        st = _lib.moer_route(*self._args)
        if st != MOER_OK:
            _check(st)


def moer_load_stats(counts, n_layers, N, stride, out, stream=None):
    """out: uint8 device tensor of n_layers*64 bytes (moer_load_stats_t records)."""
    if counts.dtype != torch.int32:
        raise TypeError("counts must be int32")
    if out.numel() * out.element_size() < 64 * n_layers:
        raise ValueError("out needs 64 bytes per layer")
    _check(_lib.moer_load_stats(_ptr(counts), n_layers, N, stride, _ptr(out), _stream(stream)))


def moer_bias_update(bias, counts, n_layers, N, stride, u, stream=None):
    if bias.dtype != torch.float32 or counts.dtype != torch.int32:
        raise TypeError("bias must be float32 and counts int32")
    _check(_lib.moer_bias_update(_ptr(bias), _ptr(counts), n_layers, N, stride, u,
                                 _stream(stream)))


_DTYPE_CODE = {torch.bfloat16: MOER_BF16, torch.float32: MOER_F32}


def moer_dispatch(x, row_bytes, n_layers, T, Kt, inv_perm, x_out, stream=None):
    """x [L,T,...] rows of row_bytes bytes -> x_out [L,T*Kt,...] in layout
    order (rows no slot names are left as they are)."""
    if inv_perm.dtype != torch.int32:
        raise TypeError("inv_perm must be int32")
    if x.dtype != x_out.dtype:
        raise TypeError("x and x_out must have the same dtype")
    _check(_lib.moer_dispatch(_ptr(x), int(row_bytes), n_layers, T, Kt, _ptr(inv_perm),
                              _ptr(x_out), _stream(stream)))


def moer_combine(expert_out, w, inv_perm, n_layers, T, Kt, d, y, stream=None):
    """y [L,T,d] = per token the w-weighted sum of its slots' rows of
    expert_out [L,T*Kt,d]; expert_out and y are bf16 or fp32."""
    if w.dtype != torch.float32 or inv_perm.dtype != torch.int32:
        raise TypeError("w must be float32 and inv_perm int32")
    if expert_out.dtype not in _DTYPE_CODE or y.dtype not in _DTYPE_CODE:
        raise TypeError("expert_out and y must be bfloat16 or float32")
    _check(_lib.moer_combine(_ptr(expert_out), _DTYPE_CODE[expert_out.dtype], _ptr(w),
                             _ptr(inv_perm), n_layers, T, Kt, d, _ptr(y), _DTYPE_CODE[y.dtype],
                             _stream(stream)))


def moer_balance_step(bias, counts, n_layers, N, stride, cfg, loads=None, calls=None,
                      stream=None):
    """cfg: MoerBalanceCfg; loads [L,N] fp32 and calls [L] int32 are the
    caller's state (device tensors or None)."""
    if bias.dtype != torch.float32 or counts.dtype != torch.int32:
        raise TypeError("bias must be float32 and counts int32")
    if loads is not None and loads.dtype != torch.float32:
        raise TypeError("loads must be float32")
    if calls is not None and calls.dtype != torch.int32:
        raise TypeError("calls must be int32")
    _check(_lib.moer_balance_step(_ptr(bias), _ptr(counts), n_layers, N, stride,
                                  ctypes.byref(cfg), _ptr(loads), _ptr(calls), _stream(stream)))


def moer_balanced_indices(idx, n_layers, T, K, N, n_shared=0, first=0, stream=None):
    if idx.dtype != torch.int32:
        raise TypeError("idx must be int32")
    _check(_lib.moer_balanced_indices(_ptr(idx), n_layers, T, K, N, n_shared, int(first),
                                      _stream(stream)))


def moer_hotspot_accumulate(hot, counts, n_layers, N, stride, stream=None):
    if hot.dtype != torch.int64 or counts.dtype != torch.int32:
        raise TypeError("hot must be int64 and counts int32")
    _check(_lib.moer_hotspot_accumulate(_ptr(hot), _ptr(counts), n_layers, N, stride,
                                        _stream(stream)))


def decode_load_stats(raw):
    """Host view of moer_load_stats_t records (raw: CPU uint8 tensor)."""
    b = bytes(raw.contiguous().numpy().tobytes())
    out = []
    for i in range(len(b) // 64):
        rec = MoerLoadStats.from_buffer_copy(b[i * 64:(i + 1) * 64])
        out.append({n: getattr(rec, n) for n in LOAD_STATS_FIELDS})
    return out
