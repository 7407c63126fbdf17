"""moer_route captured once in a HIP graph and replayed (GPU): every replay
rewrites every output exactly as the eager call does.

The call clears its own counters with fill kernels (no memset nodes), so a
captured call must be replayable any number of times. Between replays the
program does eager work of its own: the outputs are overwritten with a
sentinel, an eager route runs on another stream into other buffers, and
everything is synchronised; then each replay's outputs are compared with the
eager call's bit for bit. No bias update is asked for, so every call does the
same work. Shapes: the DeepSeek-V3 router (split-K GEMM, 64-token
selection), a one-layer decode batch (small GEMM tile, 16-token selection),
the top-2-of-8 router (one-launch GEMM + selection), the same router at 20
tokens (one workgroup per layer that also writes the layout), several
layers, and a capacity-limited route (its rounds of proposals, ranking and
re-layout).
"""
import pytest
import torch

import top_expert_routing_gate_amd as moer
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
WL = workloads.WORKLOADS

CASES = [
    ("dsv3", workloads.scaled(WL["dsv3_group"], T=2048), 0),
    ("decode_one_layer", workloads.scaled(WL["decode_layers"], n_layers=1), 0),
    ("mixtral", workloads.scaled(WL["mixtral_top2"], T=1024), 0),
    ("mixtral_whole_layer", workloads.scaled(WL["mixtral_top2"], T=20, d=256), 0),
    ("decode_layers", workloads.scaled(WL["decode_layers"], n_layers=4, T=100), 0),
    ("capacity", workloads.scaled(WL["collapse_balance"], T=1024, d=1024), 20),
]


def _buffers(wl, L, T, capacity):
    i32 = dict(dtype=torch.int32, device=DEV)
    f32 = dict(dtype=torch.float32, device=DEV)
    Kt, Nb = wl.Kt, wl.Nb
    out = dict(topk_idx=torch.empty(L, T, Kt, **i32), topk_w=torch.empty(L, T, Kt, **f32),
               tok_entropy=torch.empty(L, T, **f32), agg_entropy=torch.empty(L, **f32),
               counts=torch.empty(L, Nb, **i32), offsets=torch.empty(L, Nb + 1, **i32),
               perm=torch.empty(L, T * Kt, **i32), inv_perm=torch.empty(L, T * Kt, **i32),
               h_out=torch.empty(L, T, wl.N, **f32),
               load_stats=torch.empty(L, 64, dtype=torch.uint8, device=DEV))
    if capacity > 0:  # written only by a capacity-limited call
        out["cap_stats"] = torch.empty(L, 2, **i32)
    return out


@pytest.mark.parametrize("name,wl,capacity", CASES, ids=[c[0] for c in CASES])
def test_graph_replays_equal_the_eager_call(name, wl, capacity):
    print(f"[graph] {name}: L={wl.n_layers} T={wl.T} d={wl.d} N={wl.N} capacity={capacity}",
          flush=True)
    inp = workloads.make_inputs(wl)
    L, T = wl.n_layers, wl.T
    x, W, b = inp["x"].to(DEV), inp["W"].to(DEV), inp["bias"].to(DEV)
    off = None if inp["offset"] is None else inp["offset"].to(DEV)
    desc = moer.make_desc(n_layers=L, T=T, d=wl.d, N=wl.N, K=wl.K, n_groups=wl.n_groups,
                          topk_groups=wl.topk_groups, n_shared=wl.n_shared,
                          score_fn=wl.score_fn, dtype=wl.dtype, capacity=capacity)
    nbytes = max(1, moer.moer_route_workspace_bytes(desc))
    eager_s, graph_s = torch.cuda.Stream(), torch.cuda.Stream()
    eager_out, graph_out, other_out = (_buffers(wl, L, T, capacity) for _ in range(3))
    eager = moer.PreparedRoute(desc, workspace=torch.empty(nbytes, dtype=torch.uint8, device=DEV),
                               stream=eager_s, x=x, w_gate=W, bias=b, logit_offset=off,
                               **eager_out)
    other = moer.PreparedRoute(desc, workspace=torch.empty(nbytes, dtype=torch.uint8, device=DEV),
                               stream=eager_s, x=x, w_gate=W, bias=b, logit_offset=off,
                               **other_out)
    captured = moer.PreparedRoute(desc,
                                  workspace=torch.empty(nbytes, dtype=torch.uint8, device=DEV),
                                  stream=graph_s, x=x, w_gate=W, bias=b, logit_offset=off,
                                  **graph_out)
    eager()
    with torch.cuda.stream(graph_s):
        captured()  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=graph_s):
        captured()
    torch.cuda.synchronize()
    for rep in range(4):
        for t in graph_out.values():
            t.fill_(-7 if t.dtype != torch.uint8 else 0xA5)
        other()  # eager work of the program's own between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, t in eager_out.items():
            assert torch.equal(graph_out[k], t), f"replay {rep}: {k} differs from the eager call"
        for k, t in eager_out.items():
            assert torch.equal(other_out[k], t), f"{k}: eager calls differ"
    del g
