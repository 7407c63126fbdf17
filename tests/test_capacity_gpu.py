"""GPU parity of capacity-limited routing (through the C ABI) against the
CPU oracle. In SCORES mode (the oracle's fp32 scores given to both sides)
the final ids, the reroute/drop counts and the layout are bit-exact, and the
weights within 1e-6 relative; in HIDDEN mode the capacity invariants are
checked on the GPU's own decisions."""
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


def _skewed_scores(wl, seed, hot=(2, 4, 7, 12), boost=3.0):
    """Oracle scores of N(0,1) logits with a few experts boosted (the
    collapse workload's celebrity offset), so capacities overflow."""
    logits = workloads.make_logits(wl.T, wl.N, seed, n_layers=wl.n_layers).double().numpy()
    logits[..., [h for h in hot if h < wl.N]] += boost
    return np.stack([oracle.scores(logits[l], wl.score_fn).astype(np.float32)
                     for l in range(wl.n_layers)])


CASES = [
    # (workload, capacity or None for the pages' 1.25 x T*K/N, boost)
    (workloads.scaled(WL["tiny_softmax"]), None, 1.0),
    (workloads.scaled(WL["mixtral_top2"], T=1500), None, 1.0),
    (workloads.scaled(WL["dsv3_group"], T=2000), None, 3.0),
    (workloads.scaled(WL["dsv3_group"], T=777), 9, 3.0),              # tight: drops
    (workloads.scaled(WL["decode_layers"], n_layers=4), None, 3.0),   # shared slot
    (workloads.scaled(WL["dsv3_group"], T=300, N=64, n_groups=1, topk_groups=1, K=4), None, 2.0),
    # group geometries of the one-wave-per-token selection kernel: groups of 4
    # (two whole lanes each), of 12 and of 20 (scored through LDS)
    (workloads.scaled(WL["dsv3_group"], T=640, N=128, n_groups=32, topk_groups=8), None, 3.0),
    (workloads.scaled(WL["dsv3_group"], T=900, N=96, n_groups=8, topk_groups=4, K=6), None, 3.0),
    (workloads.scaled(WL["dsv3_group"], T=700, N=200, n_groups=10, topk_groups=3), 40, 3.0),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0].name}-T{c[0].T}-cap{c[1]}")
def test_capacity_scores_mode_bit_exact(case):
    wl, cap, boost = case
    cap = cap or moer.expert_capacity(wl.T, wl.K, wl.N)
    say(f"[capacity] {wl.name} L={wl.n_layers} T={wl.T} N={wl.N} K={wl.K} cap={cap}")
    s32 = _skewed_scores(wl, seed=wl.T + 3, boost=boost)
    bias = workloads.make_bias(wl.N, 5, wl.bias_range, wl.n_layers) if wl.bias_range else None
    out = moer.route(scores=torch.from_numpy(s32).to(DEV), K=wl.K, score_fn=wl.score_fn,
                     n_groups=wl.n_groups, topk_groups=wl.topk_groups, n_shared=wl.n_shared,
                     bias=None if bias is None else bias.to(DEV), capacity=cap,
                     want_load_stats=True)
    torch.cuda.synchronize()
    total_rr = 0
    for l in range(wl.n_layers):
        b = None if bias is None else bias[l].numpy()
        idx, w, rr, dr = oracle.capacity_route(s32[l], s32[l].astype(np.float64), b, wl.K, cap,
                                               wl.n_groups, wl.topk_groups, wl.n_shared)
        gi = _np(out["topk_idx"][l])
        assert (gi == idx).all(), f"layer {l}: ids differ"
        assert np.allclose(_np(out["topk_w"][l]), w, rtol=1e-6, atol=1e-7)
        assert _np(out["cap_stats"][l]).tolist() == [rr, dr]
        counts, offsets, perm, inv = oracle.layout(idx, wl.Nb)
        assert (_np(out["counts"][l]) == counts).all()
        assert (_np(out["offsets"][l]) == offsets).all()
        assert (_np(out["perm"][l]) == perm).all()
        assert (_np(out["inv_perm"][l]) == inv).all()
        assert counts[:wl.N].max() <= cap
        st = moer.decode_load_stats(out["load_stats"][l:l + 1].cpu())[0]
        ref = oracle.load_stats(counts[:wl.N])
        assert st["total"] == ref["total"] and st["max_load"] == ref["max_load"]
        total_rr += rr
    assert total_rr > 0   # the case exercises rerouting


def test_capacity_full_size_collapse():
    # The collapse workload's shape (16384 tokens, 256 experts, 8 groups,
    # top-8) with the celebrity boost: capacity 640, many rounds.
    wl = WL["collapse_balance"]
    cap = moer.expert_capacity(wl.T, wl.K, wl.N)
    say(f"[capacity/full] {wl.name} T={wl.T} cap={cap}")
    s32 = _skewed_scores(wl, seed=99)
    bias = workloads.make_bias(wl.N, 7, wl.bias_range)
    out = moer.route(scores=torch.from_numpy(s32).to(DEV), K=wl.K, n_groups=wl.n_groups,
                     topk_groups=wl.topk_groups, bias=bias.to(DEV), capacity=cap)
    torch.cuda.synchronize()
    idx, w, rr, dr = oracle.capacity_route(s32[0], s32[0].astype(np.float64), bias[0].numpy(),
                                           wl.K, cap, wl.n_groups, wl.topk_groups)
    assert (_np(out["topk_idx"][0]) == idx).all()
    assert np.allclose(_np(out["topk_w"][0]), w, rtol=1e-6, atol=1e-7)
    assert _np(out["cap_stats"][0]).tolist() == [rr, dr]
    c, o, p, inv = oracle.layout(idx, wl.Nb)
    assert (_np(out["perm"][0]) == p).all() and (_np(out["counts"][0]) == c).all()
    say(f"  rerouted {rr}, dropped {dr}, max load {c.max()}")
    assert rr > 10000 and c.max() <= cap


def test_capacity_large_enough_changes_nothing():
    wl = workloads.scaled(WL["dsv3_group"], T=1000)
    s32 = _skewed_scores(wl, seed=4, boost=0.0)
    kw = dict(K=wl.K, n_groups=wl.n_groups, topk_groups=wl.topk_groups)
    plain = moer.route(scores=torch.from_numpy(s32).to(DEV), **kw)
    capped = moer.route(scores=torch.from_numpy(s32).to(DEV), capacity=wl.T * wl.K, **kw)
    torch.cuda.synchronize()
    for k in ("topk_idx", "topk_w", "counts", "offsets", "perm", "inv_perm"):
        assert torch.equal(plain[k], capped[k]), k
    assert capped["cap_stats"].cpu().tolist() == [[0, 0]]


def test_capacity_hidden_mode_invariants():
    # HIDDEN mode, the collapse workload scaled: the capacity holds, the first
    # min(cap, demand) plain assignments of every expert are kept at their
    # slots, weights renormalise over placed slots, and the reroute count
    # equals the slots that moved.
    wl = workloads.scaled(WL["collapse_balance"], T=2048, d=1024)
    cap = moer.expert_capacity(wl.T, wl.K, wl.N)
    say(f"[capacity/hidden] T={wl.T} cap={cap}")
    inp = workloads.make_inputs(wl)
    kw = dict(K=wl.K, n_groups=wl.n_groups, topk_groups=wl.topk_groups,
              bias=inp["bias"].to(DEV), logit_offset=inp["offset"].to(DEV))
    x, W = inp["x"].to(DEV), inp["W"].to(DEV)
    plain = moer.route(x, W, **kw)
    capped = moer.route(x, W, capacity=cap, **kw)
    torch.cuda.synchronize()
    pi, ci = _np(plain["topk_idx"][0]), _np(capped["topk_idx"][0])
    cw = _np(capped["topk_w"][0])
    counts = np.bincount(ci[ci >= 0], minlength=wl.N)
    assert counts.max() <= cap
    for e in range(wl.N):
        ts, ks = np.nonzero(pi == e)
        keep = np.lexsort((ks, ts))[:cap]
        assert (ci[ts[keep], ks[keep]] == e).all()
    for t in range(wl.T):
        placed = ci[t][ci[t] >= 0]
        assert len(set(placed.tolist())) == len(placed)
        assert abs(cw[t][ci[t] >= 0].sum() - 1.0) < 1e-5
    moved = int(((ci != pi) & (ci >= 0)).sum())
    dropped = int((ci < 0).sum())
    assert _np(capped["cap_stats"][0]).tolist() == [moved, dropped]
    assert moved > 0


def test_capacity_only_some_layers_overflow():
    # layer 0 skewed (experts over capacity), layer 1 forcibly balanced (every
    # expert exactly T*K/N, under the capacity), layer 2 skewed again: the
    # capacity kernels must rework layers 0 and 2 and leave layer 1 as routed
    wl = workloads.scaled(WL["dsv3_group"], T=1024, n_layers=3, n_groups=1, topk_groups=1)
    cap = moer.expert_capacity(wl.T, wl.K, wl.N)
    s32 = _skewed_scores(wl, seed=21)
    bal = np.full((wl.T, wl.N), 0.1, dtype=np.float32)
    for t in range(wl.T):
        for k in range(wl.K):
            bal[t, (t * wl.K + k) % wl.N] = 0.9 - 0.01 * k
    s32[1] = bal
    say(f"[capacity/mixed layers] T={wl.T} N={wl.N} K={wl.K} cap={cap}")
    b0 = workloads.make_bias(wl.N, 3, 0.01, wl.n_layers)
    bias = b0.clone().to(DEV)
    out = moer.route(scores=torch.from_numpy(s32).to(DEV), K=wl.K, score_fn=wl.score_fn,
                     capacity=cap, want_load_stats=True, bias_update=bias, bias_update_u=1e-3)
    plain = moer.route(scores=torch.from_numpy(s32).to(DEV), K=wl.K, score_fn=wl.score_fn)
    torch.cuda.synchronize()
    # statistics and the sign step from the final (capacity-limited) counts,
    # applied once per layer
    for l in range(wl.n_layers):
        ids = _np(out["topk_idx"][l]).ravel()
        final = np.bincount(ids[ids >= 0], minlength=wl.N)[:wl.N]
        st = moer.decode_load_stats(out["load_stats"][l:l + 1].cpu())[0]
        ref = oracle.load_stats(final)
        assert st["total"] == ref["total"] and st["max_load"] == ref["max_load"]
        expect = oracle.bias_update(b0[l].numpy(), final, 1e-3)
        assert np.array_equal(_np(bias[l]), np.asarray(expect, dtype=np.float32)), f"layer {l}"

    for l in range(wl.n_layers):
        idx, w, rr, dr = oracle.capacity_route(s32[l], s32[l].astype(np.float64), None, wl.K,
                                               cap, 1, 1, 0)
        assert (_np(out["topk_idx"][l]) == idx).all(), f"layer {l}: ids differ"
        assert np.allclose(_np(out["topk_w"][l]), w, rtol=1e-6, atol=1e-7)
        assert _np(out["cap_stats"][l]).tolist() == [rr, dr]
        counts, offsets, perm, inv = oracle.layout(idx, wl.Nb)
        assert (_np(out["perm"][l]) == perm).all() and (_np(out["inv_perm"][l]) == inv).all()
        assert counts.max() <= cap
    assert _np(out["cap_stats"][1]).tolist() == [0, 0]
    for key in ("topk_idx", "topk_w", "perm", "inv_perm", "counts", "offsets"):
        assert torch.equal(out[key][1], plain[key][1]), f"layer 1 {key} changed"
    assert _np(out["cap_stats"][0])[0] > 0 and _np(out["cap_stats"][2])[0] > 0
