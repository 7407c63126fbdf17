"""MI355X-native Mixture-of-Experts router (gfx950 HIP kernels behind a C ABI).

The C-ABI entry points (include/moer.h) are re-exported under their own names
(``moer_route``, ``moer_load_stats``, ``moer_bias_update``, ``moer_dispatch``,
``moer_combine``, ...). ``route``, ``load_stats``, ``bias_update``, ``dispatch``
and ``combine`` are conveniences that allocate the output tensors with torch
and pass the current stream; all routing work runs in the library's kernels.
"""
import torch

from ._moer import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    LOAD_STATS_FIELDS,
    MOER_BF16,
    MOER_BIAS_LOGIT,
    MOER_BIAS_SCORE,
    MOER_EHIP,
    MOER_EINVAL,
    MOER_EUNSUPPORTED,
    MOER_EWORKSPACE,
    MOER_F32,
    MOER_IN_HIDDEN,
    MOER_IN_INDICES,
    MOER_IN_SCORES,
    MOER_MAX_EXPERTS,
    MOER_MAX_SLOTS,
    MOER_OK,
    MOER_RULE_PROPORTIONAL,
    MOER_RULE_SIGN,
    MOER_SIGMOID,
    MOER_SOFTMAX,
    MoerBalanceCfg,
    MoerError,
    MoerRouteDesc,
    PreparedRoute,
    decode_load_stats,
    make_desc,
    moer_abi_version,
    moer_balance_step,
    moer_balanced_indices,
    moer_bias_update,
    moer_combine,
    moer_dispatch,
    moer_hotspot_accumulate,
    moer_load_stats,
    moer_route,
    moer_route_noalloc,
    moer_route_workspace_bytes,
    MOER_NOALLOC_SCRATCH_BYTES,
)

_SCORE_FN = {"softmax": MOER_SOFTMAX, "sigmoid": MOER_SIGMOID}
_BIAS_MODE = {"score": MOER_BIAS_SCORE, "logit": MOER_BIAS_LOGIT}
_RULE = {"sign": MOER_RULE_SIGN, "proportional": MOER_RULE_PROPORTIONAL}


def _layers(t, rank):
    """View a [T,...] tensor as [1,T,...] (a single router layer)."""
    return t if t is None or t.dim() == rank else t.unsqueeze(0)


def route(x=None, w_gate=None, *, K, score_fn="sigmoid", n_groups=1, topk_groups=1, n_shared=0,
          bias=None, logit_offset=None, scores=None, idx_in=None, N=None, want_h=False,
          want_inv_perm=True, want_entropy=True, want_load_stats=False, bias_update=None,
          bias_update_u=1e-3, bias_mode="score", capacity=0, workspace=None, stream=None):
    """Route a batch; returns a dict of device tensors, each with a leading
    layer dimension L.

    Input (one of): x [L,T,d] with w_gate [L,N,d] (bf16 or fp32), scores
    [L,T,N] fp32, or idx_in [L,T,K+n_shared] int32 (N must then be given).
    want_load_stats adds the raw load-statistics records ("load_stats", uint8
    [L,64]); bias_update [L,N] fp32 (may be `bias` itself) gets the sign-step
    update with step bias_update_u from this call's counts, in place.
    bias_mode "score" adds the bias to the scores for the selection only;
    "logit" (hidden-state input) adds it to the logits, so the weights and
    entropies come from the compensated scores too.
    capacity > 0 limits every routed expert to that many assignments per
    layer (see expert_capacity); the result then holds "cap_stats" [L, 2]
    (slots rerouted, slots dropped).
    """
    x, w_gate = _layers(x, 3), _layers(w_gate, 3)
    scores, idx_in, bias = _layers(scores, 3), _layers(idx_in, 3), _layers(bias, 2)
    bias_update = _layers(bias_update, 2)
    if x is not None:
        if w_gate is None:
            raise ValueError("x needs w_gate")
        if x.dim() != 3 or w_gate.dim() != 3:
            raise ValueError("x must be [L,T,d] and w_gate [L,N,d]")
        if w_gate.shape[0] != x.shape[0] or w_gate.shape[2] != x.shape[2]:
            raise ValueError(f"w_gate {tuple(w_gate.shape)} does not match x {tuple(x.shape)} "
                             "(need [L,N,d] for x [L,T,d])")
        mode, (L, T, d), N = MOER_IN_HIDDEN, x.shape, w_gate.shape[1]
        dev = x.device
        dtype = MOER_BF16 if x.dtype == torch.bfloat16 else MOER_F32
    elif scores is not None:
        mode, (L, T, N), d, dev, dtype = MOER_IN_SCORES, scores.shape, 0, scores.device, MOER_BF16
    else:
        mode, (L, T, _), d, dev, dtype = MOER_IN_INDICES, idx_in.shape, 0, idx_in.device, MOER_BF16
        if N is None:
            raise ValueError("N is required with idx_in")
    Kt, Nb = K + n_shared, N + n_shared
    for name, t in (("bias", bias), ("bias_update", bias_update)):
        if t is not None and tuple(t.shape) != (L, N):
            raise ValueError(f"{name} must be [L,N] = [{L},{N}], got {tuple(t.shape)}")
    if logit_offset is not None and tuple(logit_offset.shape) != (N,):
        raise ValueError(f"logit_offset must be [N] = [{N}], got {tuple(logit_offset.shape)}")
    if scores is not None and scores.dim() != 3:
        raise ValueError("scores must be [L,T,N]")
    if idx_in is not None and tuple(idx_in.shape[2:]) != (Kt,):
        raise ValueError(f"idx_in must be [L,T,K+n_shared] = [.,.,{Kt}], got {tuple(idx_in.shape)}")
    desc = make_desc(n_layers=L, T=T, d=d, N=N, K=K, n_groups=n_groups, topk_groups=topk_groups,
                     n_shared=n_shared, score_fn=_SCORE_FN.get(score_fn, score_fn), dtype=dtype,
                     input=mode, bias_mode=_BIAS_MODE.get(bias_mode, bias_mode),
                     capacity=int(capacity))
    i32, f32 = dict(dtype=torch.int32, device=dev), dict(dtype=torch.float32, device=dev)
    out = {"counts": torch.empty(L, Nb, **i32), "offsets": torch.empty(L, Nb + 1, **i32),
           "perm": torch.empty(L, T * Kt, **i32)}
    if want_inv_perm:
        out["inv_perm"] = torch.empty(L, T * Kt, **i32)
    if mode != MOER_IN_INDICES:
        out["topk_idx"] = torch.empty(L, T, Kt, **i32)
        out["topk_w"] = torch.empty(L, T, Kt, **f32)
        if want_entropy:
            out["tok_entropy"] = torch.empty(L, T, **f32)
            out["agg_entropy"] = torch.empty(L, **f32)
    if want_load_stats:
        out["load_stats"] = torch.empty(L, 64, dtype=torch.uint8, device=dev)
    if capacity:
        out["cap_stats"] = torch.empty(L, 2, **i32)
    if want_h and mode == MOER_IN_HIDDEN:
        out["h"] = torch.empty(L, T, N, **f32)
    if workspace is None:
        workspace = torch.empty(max(1, moer_route_workspace_bytes(desc)), dtype=torch.uint8,
                                device=dev)
    moer_route(desc, workspace=workspace, stream=stream, x=x, w_gate=w_gate, scores=scores,
               idx_in=idx_in, bias=bias, logit_offset=logit_offset, h_out=out.get("h"),
               topk_w=out.get("topk_w"), tok_entropy=out.get("tok_entropy"),
               agg_entropy=out.get("agg_entropy"), topk_idx=out.get("topk_idx"),
               counts=out["counts"], offsets=out["offsets"], perm=out["perm"],
               inv_perm=out.get("inv_perm"), load_stats=out.get("load_stats"),
               bias_update=bias_update, bias_update_u=bias_update_u,
               cap_stats=out.get("cap_stats"))
    return out


def expert_capacity(T, K, N, factor="1.25"):
    """Per-expert capacity ceil(factor * T * K / N) (dailyaiworld, production
    testing: 1.25 x batch x top-k / experts), in exact rational arithmetic."""
    from fractions import Fraction
    q = Fraction(factor) * T * K / N
    return -((-q.numerator) // q.denominator)


def load_stats(counts, N, stream=None):
    """Load statistics of counts [L, stride] over the first N columns; returns
    the raw device records (uint8 [L, 64])."""
    counts = _layers(counts, 2)
    L, stride = counts.shape
    out = torch.empty(L, 64, dtype=torch.uint8, device=counts.device)
    moer_load_stats(counts, L, N, stride, out, stream)
    return out


def bias_update(bias, counts, u=1e-3, stream=None):
    """In-place sign-step update of bias [L, N] from counts [L, stride]."""
    bias2, counts2 = _layers(bias, 2), _layers(counts, 2)
    moer_bias_update(bias2, counts2, bias2.shape[0], bias2.shape[1], counts2.shape[1], u, stream)
    return bias


def _rows(t, rank):
    return t if t.dim() == rank else t.unsqueeze(0)


def dispatch(x, inv_perm, Kt, out=None, stream=None):
    """Gather token rows into the layout's expert-contiguous order.

    x [L,T,d] (any dtype; rows are copied as bytes), inv_perm [L,T*Kt] as
    returned by ``route``; returns out [L,T*Kt,d] (allocated when None; rows
    no slot names are left as they are, i.e. uninitialised in a new tensor).
    """
    x, inv_perm = _rows(x, 3), _rows(inv_perm, 2)
    L, T, d = x.shape
    if out is None:
        out = torch.empty(L, T * Kt, d, dtype=x.dtype, device=x.device)
    moer_dispatch(x, d * x.element_size(), L, T, Kt, inv_perm, out, stream)
    return out


def combine(expert_out, w, inv_perm, out_dtype=torch.bfloat16, out=None, stream=None):
    """Weighted combine back to token order: y[l,t] = sum_k w[l,t,k] *
    expert_out[l, inv_perm[l, t*Kt+k]] (fp32 accumulation, one rounding).

    expert_out [L,T*Kt,d] bf16/fp32, w [L,T,Kt] fp32; returns y [L,T,d].
    """
    expert_out, w, inv_perm = _rows(expert_out, 3), _rows(w, 3), _rows(inv_perm, 2)
    L, T, Kt = w.shape
    d = expert_out.shape[2]
    if out is None:
        out = torch.empty(L, T, d, dtype=out_dtype, device=expert_out.device)
    moer_combine(expert_out, w, inv_perm, L, T, Kt, d, out, stream)
    return out


def balanced_indices(T, K, N, *, n_layers=1, n_shared=0, first=0, device="cuda", stream=None):
    """Forcible-balance expert ids [L, T, K + n_shared] int32 on the device
    (slot k of token t -> expert (t*K + k + first) mod N), for moer_route's
    INDICES mode."""
    idx = torch.empty(n_layers, T, K + n_shared, dtype=torch.int32, device=device)
    moer_balanced_indices(idx, n_layers, T, K, N, n_shared, first, stream)
    return idx


class HotspotRecorder:
    """Per-layer, per-expert token counts summed over batches (the hotspot
    matrix), kept on the device; ``write_csv`` appends the matrix (one row
    per layer, one column per expert) to a CSV file on the host."""

    def __init__(self, n_layers, N, device="cuda"):
        self.N = N
        self.hot = torch.zeros(n_layers, N, dtype=torch.int64, device=device)
        self.batches = 0

    def add(self, counts, stream=None):
        counts = _layers(counts, 2)
        moer_hotspot_accumulate(self.hot, counts, counts.shape[0], self.N, counts.shape[1], stream)
        self.batches += 1

    def write_csv(self, path):
        m = self.hot.cpu().tolist()
        with open(path, "a") as f:
            for row in m:
                f.write(",".join(str(v) for v in row) + "\n")
        return m


class BalanceState:
    """Caller-owned state of moer_balance_step for L layers of N experts:
    the moving-average loads and the per-layer call counters (zeroed)."""

    def __init__(self, n_layers, N, device="cuda"):
        self.loads = torch.zeros(n_layers, N, dtype=torch.float32, device=device)
        self.calls = torch.zeros(n_layers, dtype=torch.int32, device=device)


def balance_step(bias, counts, *, rule="sign", step=1e-3, alpha=1.0, every=1, state=None,
                 stream=None):
    """One balancing step on bias [L, N] (in place) from counts [L, stride]:
    rule "sign" (b += step*sign(mean - load)) or "proportional"
    (b -= step*(load - mean)/mean), loads smoothed by a moving average of
    weight alpha, the rule applied every `every` calls (state: a
    BalanceState, needed when alpha < 1 or every > 1)."""
    bias2, counts2 = _layers(bias, 2), _layers(counts, 2)
    cfg = MoerBalanceCfg(_RULE.get(rule, rule), float(step), float(alpha), int(every))
    moer_balance_step(bias2, counts2, bias2.shape[0], bias2.shape[1], counts2.shape[1], cfg,
                      None if state is None else state.loads,
                      None if state is None else state.calls, stream)
    return bias


class BalanceMonitor:
    """Balance alarms on the device's load statistics (hotdry, deployment
    section: keep the spread of expert activation frequency within 20 % of
    the mean; an expert whose load stays more than 50 % above the mean calls
    for a replica or a different bias step).

    ``observe(stats, counts)`` takes one layer's load-statistics record of a
    batch (from ``load_stats`` or ``route(..., want_load_stats=True)``: the
    raw uint8 [64] record or its ``decode_load_stats`` dict) and that batch's
    expert counts [N], and returns the alarms raised: ("spread", cv) when the
    record's coefficient of variation exceeds ``cv_limit``, and ("hot",
    expert, batches) for each expert whose count exceeds (1 + hot_margin) x
    the record's mean for ``persist`` consecutive batches. Only the
    thresholds and the streaks are kept on the host."""

    def __init__(self, N, cv_limit=0.20, hot_margin=0.50, persist=3):
        self.N, self.cv_limit, self.hot_margin, self.persist = N, cv_limit, hot_margin, persist
        self.streak = [0] * N

    def observe(self, stats, counts):
        if not isinstance(stats, dict):
            stats = decode_load_stats(stats.reshape(1, 64).cpu())[0]
        c = counts.tolist() if hasattr(counts, "tolist") else list(counts)
        c = c[:self.N]
        alarms = []
        if stats["total"] == 0:
            self.streak = [0] * self.N
            return alarms
        if stats["cv"] > self.cv_limit:
            alarms.append(("spread", stats["cv"]))
        limit = (1.0 + self.hot_margin) * stats["mean"]
        for e, v in enumerate(c):
            self.streak[e] = self.streak[e] + 1 if v > limit else 0
            if self.streak[e] >= self.persist:
                alarms.append(("hot", e, self.streak[e]))
        return alarms
