"""moer_route_noalloc (the allocation-free variant of moer_route, whose
scratch is the library's static per-GPU array) against moer_route with a
caller workspace, through the C ABI: every output bitwise equal, on calls in
a row, each with a smaller batch than the one before (so each runs on the
previous call's leftover scratch contents): the 16k-token batch, a 3-layer
decode batch, a 300-token top-2-of-8 batch (the one-launch small-router
kernel and its layout launch) and a 20-token one (one workgroup per layer
that also writes the layout)."""
import numpy as np
import pytest
import torch

import top_expert_routing_gate_amd as moer
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _buffers(wl):
    L, T, N, Kt, Nb = wl.n_layers, wl.T, wl.N, wl.Kt, wl.Nb
    i32, f32 = dict(dtype=torch.int32, device=DEV), dict(dtype=torch.float32, device=DEV)
    return dict(topk_idx=torch.full((L, T, Kt), -7, **i32),
                topk_w=torch.full((L, T, Kt), -7.0, **f32),
                tok_entropy=torch.full((L, T), -7.0, **f32),
                agg_entropy=torch.full((L,), -7.0, **f32),
                counts=torch.full((L, Nb), -7, **i32), offsets=torch.full((L, Nb + 1), -7, **i32),
                perm=torch.full((L, T * Kt), -7, **i32), inv_perm=torch.full((L, T * Kt), -7, **i32),
                h_out=torch.full((L, T, N), -7.0, **f32),
                load_stats=torch.zeros(L, 64, dtype=torch.uint8, device=DEV))


def _desc(wl):
    return moer.make_desc(n_layers=wl.n_layers, T=wl.T, d=wl.d, N=wl.N, K=wl.K,
                          n_groups=wl.n_groups, topk_groups=wl.topk_groups, n_shared=wl.n_shared,
                          score_fn=wl.score_fn, dtype=wl.dtype)


def _both(wl):
    inp = workloads.make_inputs(wl)
    x, W = inp["x"].to(DEV), inp["W"].to(DEV)
    off = None if inp["offset"] is None else inp["offset"].to(DEV)
    desc = _desc(wl)
    outs = []
    for noalloc in (True, False):
        bias = inp["bias"].to(DEV)  # updated in place by the call
        buf = _buffers(wl)
        kw = dict(x=x, w_gate=W, bias=bias, logit_offset=off, bias_update=bias,
                  bias_update_u=1e-3, **buf)
        if noalloc:
            moer.moer_route_noalloc(desc, **kw)
        else:
            ws = torch.empty(max(1, moer.moer_route_workspace_bytes(desc)), dtype=torch.uint8,
                             device=DEV)
            moer.moer_route(desc, workspace=ws, **kw)
        torch.cuda.synchronize()
        buf["bias_after"] = bias
        outs.append(buf)
    return outs


@pytest.mark.parametrize("order", ["large-then-small"])
def test_noalloc_matches_workspace_route_on_two_calls(order):
    first = workloads.WORKLOADS["collapse_balance"]                        # 16384 tokens
    second = workloads.scaled(workloads.WORKLOADS["decode_layers"], n_layers=3, T=100)
    # a small router: the 16-token one-launch kernel, then a layer short
    # enough for one workgroup
    third = workloads.scaled(workloads.WORKLOADS["mixtral_top2"], T=300, d=512)
    fourth = workloads.scaled(workloads.WORKLOADS["mixtral_top2"], T=20, d=256)
    for wl in (first, second, third, fourth):
        print(f"[noalloc] {wl.name} L={wl.n_layers} T={wl.T}", flush=True)
        a, b = _both(wl)
        for k in a:
            assert torch.equal(a[k], b[k]), f"{wl.name}: {k} differs"
        assert (a["counts"][:, :wl.N].sum(dim=1).cpu().numpy() == wl.T * wl.K).all()


def test_noalloc_rejects_routers_beyond_its_scratch():
    wl = workloads.WORKLOADS["dsv3_group"]
    desc = moer.make_desc(n_layers=1, T=wl.T, d=wl.d, N=wl.N, K=wl.K, n_groups=wl.n_groups,
                          topk_groups=wl.topk_groups, capacity=640)
    assert moer.moer_route_workspace_bytes(desc) > moer.MOER_NOALLOC_SCRATCH_BYTES
    with pytest.raises(moer.MoerError, match="static scratch"):
        moer.moer_route_noalloc(desc, **{k: v for k, v in _buffers(wl).items()
                                        if k not in ("h_out", "load_stats")})
