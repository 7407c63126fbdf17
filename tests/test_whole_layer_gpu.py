"""Small layers on routers with at most 16 experts (GPU): one workgroup per
layer forms the affinities, routes every token (rows of 4, 8 or 16 lanes, the
fewest that hold the router's experts) and writes the layout outputs itself
(counts, offsets, perm, inv_perm, the batch-mean entropy, load statistics and
the in-place bias update), so the call is one launch. It takes layers of at
most 64 tokens (at most 8 experts) or 32 (at most 16) with a short depth;
MOER_ROUTE_WHOLE=0 keeps the separate layout launch after the 16-token
workgroups.

Bars:
- against the CPU oracle on the same inputs: h within 1e-3, selections equal
  except where the oracle's deciding margin is below 1e-3, weights within
  1e-3, token and batch-mean entropies within 1e-4 bits, the layout bit-exact
  from the GPU's own ids, load statistics (integers exact, derived values
  1e-9 relative) and the sign-step bias update bit-exact from the GPU's
  counts, over three consecutive calls that update the bias in place;
- against the two-launch path: every output bit for bit, except the
  batch-mean entropy (within 1e-5: its column sums are associated per
  workgroup). Narrower rows change no per-token result: a row holds all of
  the router's experts (N <= RL, K <= N), so each lane holds at most one
  chosen slot, and a 16-lane row's extra lanes add exact zeros to the same
  butterfly sums.

Shapes: the fp32 toy router itself (64 tokens, 4 experts, top-1 softmax:
4-lane rows), one token (5 experts: 8-lane rows), 64 tokens of 4 experts
with 15 shared slots (1024 layout entries, the most one workgroup takes), a
bf16 top-2-of-8 router over three layers at the deepest short depth (512),
expert groups in 4-, 8- and 16-lane rows, 16 experts with shared slots, ragged
batches (17 and 31 tokens), a softmax router with 9 experts; and two shapes
past the limits (64 tokens of 16 experts; depth 1024), which keep the two
launches whatever the switch says.
"""
import numpy as np
import pytest
import torch

import oracle
import top_expert_routing_gate_amd as moer
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
WL = workloads.WORKLOADS

SHAPES = [
    WL["tiny_softmax"],
    workloads.scaled(WL["mixtral_top2"], T=1, d=384, N=5, K=3),
    workloads.scaled(WL["tiny_softmax"], T=64, d=128, N=4, K=1, n_shared=15),
    workloads.scaled(WL["mixtral_top2"], T=64, d=512, n_layers=3),
    workloads.scaled(WL["mixtral_top2"], T=48, d=256, N=8, K=2, n_groups=4, topk_groups=2),
    workloads.scaled(WL["tiny_softmax"], T=40, d=64, N=4, K=1, n_groups=2, topk_groups=1),
    workloads.scaled(WL["mixtral_top2"], T=24, d=256, N=16, K=4, n_groups=4, topk_groups=2,
                     n_shared=2),
    workloads.scaled(WL["tiny_softmax"], T=32, d=128, N=16, K=1, n_shared=15),
    workloads.scaled(WL["tiny_softmax"], T=17, d=64, N=3, K=2, n_shared=1),
    workloads.scaled(WL["tiny_softmax"], T=31, d=192, N=9, K=2),
    workloads.scaled(WL["mixtral_top2"], T=64, d=256, N=16, K=2),
    workloads.scaled(WL["mixtral_top2"], T=20, d=1024),
]
STEPS = 3
U = 2e-3


def say(msg):
    print(msg, flush=True)


def _np(t):
    return t.detach().cpu().numpy()


def _run(wl, inp, bias0):
    """STEPS calls with the bias updated in place; returns each call's outputs
    (copied) and the bias before each call."""
    x, W = inp["x"].to(DEV), inp["W"].to(DEV)
    off = None if inp["offset"] is None else inp["offset"].to(DEV)
    bias = bias0.clone().to(DEV)
    outs, biases = [], []
    for _ in range(STEPS):
        biases.append(bias.clone())
        out = moer.route(x, W, K=wl.K, score_fn=wl.score_fn, n_groups=wl.n_groups,
                         topk_groups=wl.topk_groups, n_shared=wl.n_shared, bias=bias,
                         logit_offset=off, want_h=True, want_load_stats=True,
                         bias_update=bias, bias_update_u=U)
        torch.cuda.synchronize()
        outs.append({k: v.clone() for k, v in out.items() if torch.is_tensor(v)})
    biases.append(bias.clone())
    return outs, biases


@pytest.mark.parametrize("wl", SHAPES,
                         ids=lambda w: f"{w.name}-T{w.T}-d{w.d}-N{w.N}-K{w.K}-S{w.n_shared}"
                                       f"-G{w.n_groups}-L{w.n_layers}")
def test_one_workgroup_layer_matches_oracle_and_two_launches(wl, monkeypatch):
    say(f"[whole layer] {wl}")
    inp = workloads.make_inputs(wl)
    bias0 = inp["bias"].float()
    monkeypatch.setenv("MOER_ROUTE_WHOLE", "1")
    whole, b_whole = _run(wl, inp, bias0)
    monkeypatch.setenv("MOER_ROUTE_WHOLE", "0")
    split, b_split = _run(wl, inp, bias0)

    # the two paths agree bit for bit (batch-mean entropy: association only)
    for step in range(STEPS):
        for k, u in whole[step].items():
            v = split[step][k]
            if k == "agg_entropy":
                assert torch.allclose(u, v, rtol=0, atol=1e-5), (step, k)
            else:
                assert torch.equal(u, v), f"step {step}: {k} differs from the two-launch path"
    for u, v in zip(b_whole, b_split):
        assert torch.equal(u, v), "bias updates differ"

    # against the oracle, every call
    x, W = inp["x"].float().numpy(), inp["W"].float().numpy()
    off = None if inp["offset"] is None else inp["offset"].numpy()
    for step in range(STEPS):
        out = whole[step]
        got = moer.decode_load_stats(out["load_stats"].cpu())
        for l in range(wl.n_layers):
            b = _np(b_whole[step][l])
            ref = oracle.route(x=x[l], W=W[l], offset=off, bias=b, K=wl.K, score_fn=wl.score_fn,
                               n_groups=wl.n_groups, topk_groups=wl.topk_groups,
                               n_shared=wl.n_shared)
            assert np.abs(_np(out["h"][l]).astype(np.float64) - ref["h"]).max() < 1e-3
            gi = _np(out["topk_idx"][l])
            same = (gi == ref["idx"]).all(axis=1)
            assert np.all(same | (ref["gap"] < 1e-3)), (step, l, "selection")
            gw = _np(out["topk_w"][l])
            if same.any():
                assert np.abs(gw[same] - ref["w"][same]).max() < 1e-3, (step, l, "weights")
            assert np.abs(_np(out["tok_entropy"][l]) - ref["tok_H"]).max() < 1e-4
            assert abs(float(out["agg_entropy"][l]) - ref["agg_H"]) < 1e-4, (step, l)
            counts, offsets, perm, inv = oracle.layout(gi, wl.Nb)
            assert (_np(out["counts"][l]) == counts).all(), (step, l)
            assert (_np(out["offsets"][l]) == offsets).all(), (step, l)
            assert (_np(out["perm"][l]) == perm).all(), (step, l)
            assert (_np(out["inv_perm"][l]) == inv).all(), (step, l)
            st = oracle.load_stats(counts[:wl.N])
            for k in ("total", "max_load", "argmax", "capacity"):
                assert got[l][k] == st[k], (step, l, k)
            for k in ("mean", "imbalance", "h_load_bits", "cv"):
                assert got[l][k] == pytest.approx(st[k], rel=1e-9, abs=1e-12), (step, l, k)
            nb = oracle.bias_update(b.copy(), counts[:wl.N], U)
            assert (_np(b_whole[step + 1][l]) == nb).all(), (step, l, "bias update")


# The optional outputs left out (no entropies, no inverse permutation, no
# affinities): the kernels skip those stores, and every output still asked for
# keeps its bits. The one-workgroup layer kernel in 4- and 16-lane rows, and
# the 16-token one-launch kernel with its layout launch.
@pytest.mark.parametrize("wl", [
    WL["tiny_softmax"],
    workloads.scaled(WL["mixtral_top2"], T=24, d=256, N=16, K=4, n_groups=4, topk_groups=2,
                     n_shared=2),
    workloads.scaled(WL["mixtral_top2"], T=300, d=512),
], ids=lambda w: f"{w.name}-T{w.T}-N{w.N}")
def test_optional_outputs_left_out(wl):
    say(f"[whole layer, outputs left out] {wl}")
    inp = workloads.make_inputs(wl)
    kw = dict(K=wl.K, score_fn=wl.score_fn, n_groups=wl.n_groups, topk_groups=wl.topk_groups,
              n_shared=wl.n_shared, bias=inp["bias"].float().to(DEV))
    x, W = inp["x"].to(DEV), inp["W"].to(DEV)
    full = moer.route(x, W, want_h=True, want_load_stats=True, **kw)
    bare = moer.route(x, W, want_entropy=False, want_inv_perm=False, **kw)
    torch.cuda.synchronize()
    assert "tok_entropy" not in bare and "inv_perm" not in bare
    for k in ("topk_idx", "topk_w", "counts", "offsets", "perm"):
        assert torch.equal(bare[k], full[k]), k
