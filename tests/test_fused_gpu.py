"""GPU parity of the fused router pass (gate GEMM halves exchanging partial
affinities, selection from LDS, layout after a grid barrier) against the CPU
oracle, and against the separate-launch path.

The fused pass is opt-in (it is slower on MI355X than the separate launches:
its grid-wide synchronisation costs more than the kernel boundaries it
removes). MOER_ROUTE_FUSED=3 makes moer_route take it for every shape it can
(bf16, 128 < N <= 256 with N % 16 == 0, d % 128 == 0, the whole grid
resident); 1 for the 16k-token batch (two depth halves, like the separate
GEMM); 2 the same with the layout launched separately; 0 (the default) never. Bars as in test_parity_gpu.py (HIDDEN mode): h
within 1e-3 of the fp64 oracle, selections equal except where the oracle's
deciding margin is below 1e-3, weights within 1e-3, entropies within 1e-4
bits, the layout bit-exact against the oracle run on the GPU's own ids, load
statistics and the bias update against the oracle on the GPU's own counts.
Where both paths split d in two (the 16k-token batch), their outputs must be
bitwise identical apart from the batch-mean entropy's summation order.
"""
import contextlib
import os

import numpy as np
import pytest
import torch

import oracle
import top_expert_routing_gate_amd as moer
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
WL = workloads.WORKLOADS


def say(msg):
    print(msg, flush=True)


def _np(t):
    return t.detach().cpu().numpy()


@contextlib.contextmanager
def fused_mode(mode):
    old = os.environ.get("MOER_ROUTE_FUSED")
    os.environ["MOER_ROUTE_FUSED"] = str(mode)
    try:
        yield
    finally:
        if old is None:
            del os.environ["MOER_ROUTE_FUSED"]
        else:
            os.environ["MOER_ROUTE_FUSED"] = old


def _route(wl, inp, bias_mode="score", update=False):
    x, W, b, off = inp["x"], inp["W"], inp["bias"], inp["offset"]
    bias = b.to(DEV)
    out = moer.route(x.to(DEV), W.to(DEV), K=wl.K, score_fn=wl.score_fn, n_groups=wl.n_groups,
                     topk_groups=wl.topk_groups, n_shared=wl.n_shared, bias=bias,
                     logit_offset=None if off is None else off.to(DEV), want_h=True,
                     bias_mode=bias_mode, want_load_stats=True,
                     bias_update=bias if update else None, bias_update_u=1e-3)
    torch.cuda.synchronize()
    out["bias_after"] = bias
    return out


def _check_against_oracle(wl, inp, out, bias_mode="score", update=False):
    x, W, b, off = inp["x"], inp["W"], inp["bias"], inp["offset"]
    n_diff, worst = 0, 0.0
    for l in range(wl.n_layers):
        ref = oracle.route(x=x[l].float().numpy(), W=W[l].float().numpy(),
                           offset=None if off is None else off.numpy(), bias=b[l].numpy(),
                           K=wl.K, score_fn=wl.score_fn, n_groups=wl.n_groups,
                           topk_groups=wl.topk_groups, n_shared=wl.n_shared, bias_mode=bias_mode)
        gh = _np(out["h"][l]).astype(np.float64)
        dh = np.abs(gh - ref["h"]).max()
        worst = max(worst, dh)
        assert dh < 1e-3, f"layer {l}: max |dh| = {dh}"
        gi = _np(out["topk_idx"][l])
        same = (gi == ref["idx"]).all(axis=1)
        n_diff += int((~same).sum())
        assert np.all(same | (ref["gap"] < 1e-3)), "selection differs beyond the near-tie allowance"
        gw = _np(out["topk_w"][l])
        assert np.abs(gw[same] - ref["w"][same]).max() < 1e-3
        assert np.abs(_np(out["tok_entropy"][l]) - ref["tok_H"]).max() < 1e-4
        # the batch-mean entropy against the oracle's own (not the GPU's) h
        assert abs(float(out["agg_entropy"][l]) - ref["agg_H"]) < 1e-4
        counts, offsets, perm, inv = oracle.layout(gi, wl.Nb)
        assert (_np(out["counts"][l]) == counts).all()
        assert (_np(out["offsets"][l]) == offsets).all()
        assert (_np(out["perm"][l]) == perm).all()
        assert (_np(out["inv_perm"][l]) == inv).all()
        st = moer.decode_load_stats(out["load_stats"].cpu())[l]
        rs = oracle.load_stats(counts[:wl.N])
        for k in ("total", "max_load", "argmax", "capacity"):
            assert st[k] == rs[k], k
        for k in ("mean", "imbalance", "h_load_bits", "cv"):
            assert st[k] == pytest.approx(rs[k], rel=1e-9, abs=1e-12), k
        if update:
            want = oracle.bias_update(b[l].numpy(), counts[:wl.N], 1e-3)
            assert (_np(out["bias_after"][l]) == want).all(), "bias update differs"
    return n_diff, worst


FUSED_SHAPES = [
    workloads.scaled(WL["dsv3_group"], T=1000, d=1024),
    workloads.scaled(WL["dsv3_group"], T=64, d=128),
    workloads.scaled(WL["collapse_balance"], T=777, d=1024),
    workloads.scaled(WL["decode_layers"], n_layers=2, T=4097, d=512),
    workloads.scaled(WL["dsv3_group"], T=333, d=256, N=192, n_groups=6, topk_groups=2, K=6),
    workloads.scaled(WL["dsv3_group"], T=129, d=384, N=144, n_groups=9, topk_groups=3, K=4,
                     score_fn=oracle.SOFTMAX),
    workloads.scaled(WL["dsv3_group"], T=500, d=1024, N=256, n_groups=4, topk_groups=2, K=8,
                     score_fn=oracle.SOFTMAX),
    workloads.scaled(WL["dsv3_group"], T=250, d=256, N=160, n_groups=1, topk_groups=1, K=16),
]


@pytest.mark.parametrize("wl", FUSED_SHAPES,
                         ids=lambda w: f"{w.name}-L{w.n_layers}-T{w.T}-d{w.d}-N{w.N}-G{w.n_groups}")
def test_fused_pass_matches_oracle(wl):
    say(f"[fused] {wl}")
    inp = workloads.make_inputs(wl)
    with fused_mode(3):
        out = _route(wl, inp, update=True)
    n_diff, worst = _check_against_oracle(wl, inp, out, update=True)
    say(f"  max|dh|={worst:.2e}, near-tie differences={n_diff}")


@pytest.mark.parametrize("wl", [workloads.scaled(WL["dsv3_group"], T=900, d=512),
                                workloads.scaled(WL["collapse_balance"], T=300, d=1024)],
                         ids=lambda w: f"{w.name}-T{w.T}")
def test_fused_pass_logit_space_bias(wl):
    say(f"[fused/logit bias] {wl}")
    inp = workloads.make_inputs(wl)
    with fused_mode(3):
        out = _route(wl, inp, bias_mode="logit")
    _check_against_oracle(wl, inp, out, bias_mode="logit")


def test_fused_pass_empty_and_tiny():
    # one token: a single tile whose second half routes nothing
    wl = workloads.scaled(WL["dsv3_group"], T=1, d=128)
    inp = workloads.make_inputs(wl)
    with fused_mode(3):
        out = _route(wl, inp, update=True)
    _check_against_oracle(wl, inp, out, update=True)


@pytest.mark.parametrize("name", ["dsv3_group", "collapse_balance"])
def test_fused_full_size_equals_separate_launches(name):
    """The 16k-token batch: the fused pass and the separate launches (also
    two depth halves) give the same bits."""
    wl = WL[name]
    say(f"[fused/full] {wl}")
    inp = workloads.make_inputs(wl)
    with fused_mode(1):
        fused = _route(wl, inp, update=True)
    with fused_mode(0):
        sep = _route(wl, inp, update=True)
    for k in ("h", "topk_idx", "topk_w", "tok_entropy", "counts", "offsets", "perm", "inv_perm",
              "load_stats", "bias_after"):
        assert torch.equal(fused[k], sep[k]), f"{k} differs between the fused and separate paths"
    assert abs(float(fused["agg_entropy"][0]) - float(sep["agg_entropy"][0])) < 1e-5
    n_diff, worst = _check_against_oracle(wl, inp, fused, update=True)
    say(f"  all {wl.T} tokens: max|dh|={worst:.2e}, near-tie differences={n_diff}")


def test_fused_layout_as_separate_launch():
    """Mode 2 (fused GEMM and selection, the layout as its own launch) gives
    the fully fused pass's bits on the 16k-token batch (the batch-mean
    entropy is summed in another order)."""
    wl = WL["dsv3_group"]
    inp = workloads.make_inputs(wl)
    with fused_mode(2):
        a = _route(wl, inp, update=True)
    with fused_mode(1):
        b = _route(wl, inp, update=True)
    for k in ("h", "topk_idx", "topk_w", "tok_entropy", "counts", "offsets", "perm", "inv_perm",
              "load_stats", "bias_after"):
        assert torch.equal(a[k], b[k]), k
    assert abs(float(a["agg_entropy"][0]) - float(b["agg_entropy"][0])) < 1e-5


def test_fused_pass_is_deterministic_and_ignores_workspace_contents():
    wl = workloads.scaled(WL["dsv3_group"], T=3000, d=512)
    inp = workloads.make_inputs(wl)
    desc = moer.make_desc(n_layers=1, T=wl.T, d=wl.d, N=wl.N, K=wl.K, n_groups=wl.n_groups,
                          topk_groups=wl.topk_groups, n_shared=0, score_fn=moer.MOER_SIGMOID,
                          dtype=moer.MOER_BF16, input=moer.MOER_IN_HIDDEN)
    nbytes = moer.moer_route_workspace_bytes(desc)
    outs = []
    with fused_mode(3):
        for fill in (0, 255, 7):
            ws = torch.full((nbytes,), fill, dtype=torch.uint8, device=DEV)
            o = moer.route(inp["x"].to(DEV), inp["W"].to(DEV), K=wl.K, score_fn=wl.score_fn,
                           n_groups=wl.n_groups, topk_groups=wl.topk_groups,
                           bias=inp["bias"].to(DEV), want_h=True, workspace=ws)
            torch.cuda.synchronize()
            outs.append(o)
    for o in outs[1:]:
        for k in o:
            assert torch.equal(o[k], outs[0][k]), k
