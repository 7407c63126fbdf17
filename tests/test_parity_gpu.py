"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (fixed by the router's specification):
 - SCORES mode (fp32 scores given): expert ids, counts, offsets, perm and
   inv_perm bit-exact; weights within 1e-6 relative; entropies within 1e-4
   bits.
 - HIDDEN mode (bf16 x, W_g; fp32 accumulation): h within 1e-3 absolute of
   the fp64 oracle; a token's selection may differ only where the oracle's
   deciding margin is below 1e-3; weights of identical selections within
   1e-3; entropies within 1e-4 bits; the layout bit-exact against the oracle
   run on the GPU's own ids.
 - Load statistics: integers exact, derived values within 1e-9 relative;
   bias update bit-exact.
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


def say(msg):
    print(msg, flush=True)


def _np(t):
    return t.detach().cpu().numpy()


def _oracle_scores(logits, score_fn):
    s64 = oracle.scores(logits.double().numpy(), score_fn)
    return s64.astype(np.float32)


def _check_layout(out, layer, idx, Nb):
    counts, offsets, perm, inv = oracle.layout(idx, Nb)
    assert (_np(out["counts"][layer]) == counts).all()
    assert (_np(out["offsets"][layer]) == offsets).all()
    assert (_np(out["perm"][layer]) == perm).all()
    if "inv_perm" in out:
        assert (_np(out["inv_perm"][layer]) == inv).all()


def _scores_case(wl, seed, logits=None, bias=None):
    """Route oracle-made fp32 scores on the GPU and compare bit for bit."""
    L, T, N = wl.n_layers, wl.T, wl.N
    if logits is None:
        logits = workloads.make_logits(T, N, seed, n_layers=L)
    if bias is None:
        bias = workloads.make_bias(N, seed + 1, wl.bias_range, L) if wl.bias_range else None
    s32 = np.stack([_oracle_scores(logits[l], wl.score_fn) for l in range(L)])
    out = moer.route(scores=torch.from_numpy(s32).to(DEV), K=wl.K, score_fn=wl.score_fn,
                     n_groups=wl.n_groups, topk_groups=wl.topk_groups, n_shared=wl.n_shared,
                     bias=None if bias is None else bias.to(DEV))
    torch.cuda.synchronize()
    for l in range(L):
        b = None if bias is None else bias[l].numpy()
        ref = oracle.route(s32=s32[l], bias=b, K=wl.K, score_fn=wl.score_fn,
                           n_groups=wl.n_groups, topk_groups=wl.topk_groups,
                           n_shared=wl.n_shared)
        gi = _np(out["topk_idx"][l])
        assert (gi == ref["idx"]).all(), f"layer {l}: ids differ"
        gw = _np(out["topk_w"][l]).astype(np.float64)
        assert np.allclose(gw, ref["w"], rtol=1e-6, atol=1e-7)
        assert np.abs(_np(out["tok_entropy"][l]) - ref["tok_H"]).max() < 1e-4
        assert abs(float(out["agg_entropy"][l]) - ref["agg_H"]) < 1e-4
        _check_layout(out, l, ref["idx"], wl.Nb)
    return out, s32


@pytest.mark.parametrize("name", ["tiny_softmax", "mixtral_top2", "dsv3_group", "decode_layers"])
def test_scores_mode_bit_exact_full_size(name):
    wl = WL[name]
    say(f"[scores/full] {name} L={wl.n_layers} T={wl.T} N={wl.N}")
    _scores_case(wl, seed=100)


def test_scores_mode_bit_exact_many_segments():
    # 100,003 tokens: 1563 histogram blocks in 98 segments of running totals
    # (the layout sums them in chunks of 32), ragged last block
    wl = workloads.scaled(WL["dsv3_group"], T=100003)
    say(f"[scores/many segments] T={wl.T}")
    _scores_case(wl, seed=11)


@pytest.mark.parametrize("wl", [
    workloads.scaled(WL["dsv3_group"], T=1000),
    workloads.scaled(WL["mixtral_top2"], T=333),
    workloads.scaled(WL["decode_layers"], n_layers=3, T=77),
    workloads.scaled(WL["dsv3_group"], T=129, N=128, n_groups=32, topk_groups=4, K=6),
    workloads.scaled(WL["dsv3_group"], T=70, N=16, n_groups=8, topk_groups=2, K=3),
    workloads.scaled(WL["dsv3_group"], T=45, N=100, n_groups=1, topk_groups=1, K=7, n_shared=2),
    workloads.scaled(WL["dsv3_group"], T=31, N=64, n_groups=2, topk_groups=1, K=12, n_shared=4),
    workloads.scaled(WL["tiny_softmax"], T=50, N=8, K=8),
    workloads.scaled(WL["tiny_softmax"], T=3, N=1, K=1),
], ids=lambda w: f"{w.name}-T{w.T}-N{w.N}-G{w.n_groups}-K{w.K}+{w.n_shared}")
def test_scores_mode_bit_exact_ragged(wl):
    say(f"[scores/ragged] {wl}")
    _scores_case(wl, seed=7)


def _hidden_case(wl, seed_note, sample=None, check_h=True, bias_mode="score", bias=None):
    inp = workloads.make_inputs(wl)
    x, W, b, off = inp["x"], inp["W"], inp["bias"], inp["offset"]
    if bias is not None:
        b = bias
    out = moer.route(x.to(DEV), W.to(DEV), K=wl.K, score_fn=wl.score_fn, n_groups=wl.n_groups,
                     topk_groups=wl.topk_groups, n_shared=wl.n_shared, bias=b.to(DEV),
                     logit_offset=None if off is None else off.to(DEV), want_h=True,
                     bias_mode=bias_mode)
    torch.cuda.synchronize()
    worst_dh, n_diff = 0.0, 0
    for l in range(wl.n_layers):
        rows = np.arange(wl.T) if sample is None else sample
        xs = x[l][torch.from_numpy(rows)].float().numpy()
        ref = oracle.route(x=xs, W=W[l].float().numpy(), offset=None if off is None else off.numpy(),
                           bias=b[l].numpy(), K=wl.K, score_fn=wl.score_fn, n_groups=wl.n_groups,
                           topk_groups=wl.topk_groups, n_shared=wl.n_shared, bias_mode=bias_mode)
        gh = _np(out["h"][l]).astype(np.float64)
        dh = np.abs(gh[rows] - ref["h"]).max()
        worst_dh = max(worst_dh, dh)
        if check_h:
            assert dh < 1e-3, f"layer {l}: max |dh| = {dh}"
        gi = _np(out["topk_idx"][l])[rows]
        same = (gi == ref["idx"]).all(axis=1)
        n_diff += int((~same).sum())
        assert np.all(same | (ref["gap"] < 1e-3)), "selection differs beyond the near-tie allowance"
        gw = _np(out["topk_w"][l])[rows]
        assert np.abs(gw[same] - ref["w"][same]).max() < 1e-3
        assert np.abs(_np(out["tok_entropy"][l])[rows] - ref["tok_H"]).max() < 1e-4
        # layout over the whole batch from the GPU's own ids
        _check_layout(out, l, _np(out["topk_idx"][l]), wl.Nb)
        # batch-mean entropy: against the oracle's own h when every token was
        # routed by the oracle; a sampled check can only use the GPU's h
        if sample is None:
            assert abs(float(out["agg_entropy"][l]) - ref["agg_H"]) < 1e-4
        else:
            s64 = oracle.scores(gh, wl.score_fn)
            assert abs(float(out["agg_entropy"][l]) - oracle.agg_entropy(s64)) < 1e-4
    say(f"  {seed_note}: max|dh|={worst_dh:.2e}, near-tie differences={n_diff}")
    return out


@pytest.mark.parametrize("wl", [
    WL["tiny_softmax"],
    workloads.scaled(WL["decode_layers"], n_layers=1),
    workloads.scaled(WL["mixtral_top2"], T=1000),
    workloads.scaled(WL["dsv3_group"], T=700),
    workloads.scaled(WL["collapse_balance"], T=300),
    workloads.scaled(WL["decode_layers"], n_layers=3, T=100),
    workloads.scaled(WL["dsv3_group"], T=257, d=1032, N=200, n_groups=1, topk_groups=1, K=5),
    workloads.scaled(WL["dsv3_group"], T=65, d=136, N=24, n_groups=1, topk_groups=1, K=2,
                     n_shared=1),
], ids=lambda w: f"{w.name}-T{w.T}-d{w.d}-N{w.N}-L{w.n_layers}")
def test_hidden_mode_small(wl):
    say(f"[hidden/small] {wl}")
    _hidden_case(wl, wl.name)


# Routers with at most 16 experts and 4096 tokens take the one-launch gate
# GEMM + selection kernel (bf16 with d a multiple of 128, fp32 with d a
# multiple of 64); the variable MOER_ROUTE_SMALL=0 keeps them on the
# separate GEMM and selection launches.
# Shapes: depth with fewer 128-element steps than the kernel's four depth
# parts (d = 128, 384) and an odd step count, ragged token tails, one token,
# a single expert, grouped experts (16 in 4 groups of 4), shared slots,
# several layers, a logit offset (the collapse recipe's celebrity experts)
# and logit-space bias, fp32 at the depth
# limit and just past it.
SMALL_ROUTERS = [
    workloads.scaled(WL["mixtral_top2"], T=4096),
    workloads.scaled(WL["mixtral_top2"], T=77, d=128),
    workloads.scaled(WL["mixtral_top2"], T=1, d=384, N=5, K=3),
    workloads.scaled(WL["mixtral_top2"], T=200, d=4224, N=16, K=4, n_groups=4, topk_groups=2,
                     n_shared=2),
    workloads.scaled(WL["mixtral_top2"], T=130, d=640, N=1, K=1),
    workloads.scaled(WL["mixtral_top2"], T=150, d=1024, N=12, K=2, n_layers=3),
    workloads.scaled(WL["dsv3_group"], T=300, d=896, N=16, K=6, n_groups=2, topk_groups=1),
    workloads.scaled(WL["collapse_balance"], T=100, d=512, N=16, K=2, n_groups=1,
                     topk_groups=1),
    workloads.scaled(WL["tiny_softmax"], T=130, d=2048, N=16, K=3),
    workloads.scaled(WL["tiny_softmax"], T=70, d=2052, N=9, K=2),
    workloads.scaled(WL["tiny_softmax"], T=65, d=12, N=3, K=2, n_shared=1),
    workloads.scaled(WL["mixtral_top2"], T=5000, d=512),
    # the one-launch kernel's operand loads: one W_g load per step with every
    # pass two steps (4 experts, 32 steps); two W_g loads with only some
    # wavefronts taking a second step (24 steps bf16, 20 steps fp32); ragged
    workloads.scaled(WL["mixtral_top2"], T=333, d=4096, N=4, K=1),
    workloads.scaled(WL["mixtral_top2"], T=97, d=3072, N=7, K=2),
    workloads.scaled(WL["tiny_softmax"], T=90, d=1280, N=6, K=2),
]


@pytest.mark.parametrize("split", [False, True], ids=["one_launch", "split_launches"])
@pytest.mark.parametrize("wl", SMALL_ROUTERS,
                         ids=lambda w: f"{w.name}-T{w.T}-d{w.d}-N{w.N}-G{w.n_groups}-L{w.n_layers}")
def test_hidden_mode_small_routers(wl, split, monkeypatch):
    if split:
        monkeypatch.setenv("MOER_ROUTE_SMALL", "0")
    say(f"[hidden/small-router] split={split} {wl}")
    _hidden_case(wl, wl.name)
    if wl.N <= 12 and wl.n_layers == 1:
        _hidden_case(wl, wl.name + " logit-space bias", bias_mode="logit")


# Batches of fewer than 64 blocks of 64 tokens (a one-layer decode batch)
# take 16-token selection workgroups, batches of 64 to 255 blocks (the
# 64-layer decode batch, 8192 tokens) 32-token ones; MOER_ROUTE_TINY=0
# keeps them on the 64-token workgroups. Both add the same depth-range
# partials in the same order and route every row with the same routine, so
# every per-token output, the counts, the layout and the load statistics
# must be identical bit for bit. The batch-mean entropy is not: its fp32
# column sums of q are added per histogram block, and the blocks differ
# (16, 32 or 64 tokens), so only the association of the same terms differs
# (a few ulps; both paths are held to the oracle's 1e-4 elsewhere). Shapes:
# the 64-layer decode batch and an 8192-token DeepSeek-V3 batch (32-token
# workgroups), the one-layer decode batch (16 depth ranges from the gate
# GEMM's small tile), DeepSeek-V3 groups, expert counts that leave a row
# lane partly empty (200) or are not a multiple of 4 (26, with shared slots
# and a ragged d), a softmax router, several layers, one token, one-lane
# groups (16 groups of 16), three experts.
TINY_BATCHES = [
    WL["decode_layers"],
    workloads.scaled(WL["dsv3_group"], T=8192, d=1024),
    workloads.scaled(WL["decode_layers"], n_layers=1),
    workloads.scaled(WL["dsv3_group"], T=300),
    workloads.scaled(WL["dsv3_group"], T=77, d=1024, N=200, n_groups=1, topk_groups=1, K=5),
    workloads.scaled(WL["dsv3_group"], T=65, d=136, N=26, n_groups=1, topk_groups=1, K=3,
                     n_shared=2),
    workloads.scaled(WL["mixtral_top2"], T=1000, d=256, N=64, K=4),
    workloads.scaled(WL["decode_layers"], n_layers=3, T=100),
    workloads.scaled(WL["dsv3_group"], T=1, d=128),
    workloads.scaled(WL["dsv3_group"], T=130, d=256, n_groups=16, topk_groups=4),
    workloads.scaled(WL["mixtral_top2"], T=5, d=128, N=3, K=3),
]


def _route_tiny(wl, mode, inp, s32):
    if mode == "hidden":
        return moer.route(inp["x"].to(DEV), inp["W"].to(DEV), K=wl.K, score_fn=wl.score_fn,
                          n_groups=wl.n_groups, topk_groups=wl.topk_groups,
                          n_shared=wl.n_shared, bias=inp["bias"].to(DEV), want_h=True,
                          want_load_stats=True)
    return moer.route(scores=torch.from_numpy(s32).to(DEV), K=wl.K, score_fn=wl.score_fn,
                      n_groups=wl.n_groups, topk_groups=wl.topk_groups, n_shared=wl.n_shared,
                      bias=inp["bias"].to(DEV), want_load_stats=True)


@pytest.mark.parametrize("mode", ["hidden", "scores"])
@pytest.mark.parametrize("wl", TINY_BATCHES,
                         ids=lambda w: f"{w.name}-L{w.n_layers}-T{w.T}-d{w.d}-N{w.N}-G{w.n_groups}")
def test_small_batch_selection_matches_64_token_workgroups(wl, mode, monkeypatch):
    say(f"[tiny] {mode} {wl}")
    inp = workloads.make_inputs(wl)
    logits = workloads.make_logits(wl.T, wl.N, 11, n_layers=wl.n_layers)
    s32 = np.stack([_oracle_scores(logits[l], wl.score_fn) for l in range(wl.n_layers)])
    small = _route_tiny(wl, mode, inp, s32)
    monkeypatch.setenv("MOER_ROUTE_TINY", "0")
    big = _route_tiny(wl, mode, inp, s32)
    torch.cuda.synchronize()
    for k in small:
        if k == "agg_entropy":
            assert torch.allclose(small[k], big[k], rtol=0, atol=1e-5), k
        elif torch.is_tensor(small[k]):
            assert torch.equal(small[k], big[k]), f"{k} differs"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["mixtral_top2", "dsv3_group", "collapse_balance",
                                  "decode_layers"])
def test_hidden_mode_full_size_every_token(name):
    # every token of the full batch (the launch configuration the benchmark
    # times) against the oracle: h, selections (near-tie rule), weights,
    # token entropies, the batch-mean entropy of the oracle's own h, and the
    # layout of the GPU's ids
    wl = WL[name]
    say(f"[hidden/full] {name}: all {wl.n_layers} x {wl.T} tokens")
    _hidden_case(wl, name)


# ----------------------------------------------------------------- edge cases
def test_empty_batch():
    for wl in (workloads.scaled(WL["dsv3_group"], T=0, d=64),
               workloads.scaled(WL["decode_layers"], T=0, n_layers=2, d=64)):
        inp = workloads.make_inputs(wl)
        out = moer.route(inp["x"].to(DEV), inp["W"].to(DEV), K=wl.K, n_groups=wl.n_groups,
                         topk_groups=wl.topk_groups, n_shared=wl.n_shared,
                         bias=inp["bias"].to(DEV))
        torch.cuda.synchronize()
        assert (_np(out["counts"]) == 0).all() and (_np(out["offsets"]) == 0).all()
        assert (_np(out["agg_entropy"]) == 0).all()


def test_ties_and_signed_zero_scores():
    # all scores equal: groups 0..3 kept, experts 0..7 chosen, in order
    s = torch.full((1, 5, 256), 0.5)
    out = moer.route(scores=s.to(DEV), K=8, n_groups=8, topk_groups=4)
    assert (_np(out["topk_idx"][0]) == np.arange(8)).all()
    # a bias that makes two keys exactly equal: the lower id goes first
    s = torch.tensor([[[0.25, 0.5, 0.125, 0.75]]])
    b = torch.tensor([[0.5, 0.25, 0.0, 0.0]])
    out = moer.route(scores=s.to(DEV), K=3, bias=b.to(DEV))
    assert _np(out["topk_idx"][0, 0]).tolist() == [0, 1, 3]
    # -0 and +0 are the same key
    s = torch.tensor([[[-0.0, 0.0, -1.0, -2.0], [-1.0, 0.0, -0.0, -3.0]]])
    out = moer.route(scores=s.to(DEV), K=2)
    assert _np(out["topk_idx"][0]).tolist() == [[0, 1], [1, 2]]


@pytest.mark.parametrize("wl", [
    workloads.scaled(WL["dsv3_group"], T=515),
    workloads.scaled(WL["decode_layers"], T=200, n_layers=2),
    workloads.scaled(WL["mixtral_top2"], T=300),
    WL["dsv3_group"],
    workloads.scaled(WL["dsv3_group"], n_groups=1, topk_groups=1),
], ids=lambda w: f"{w.name}-T{w.T}-G{w.n_groups}")
def test_heavy_ties_quantized_scores(wl):
    """Scores drawn from a handful of values, so most tokens have dozens of
    exactly tied keys (more than the kernels rank in LDS, which sends them to
    the row-maximum rounds): ids and layout must still match the oracle bit
    for bit under (key desc, id asc). The 16k-token batches take the 64-token
    selection kernels (the DeepSeek-V3 shape's own, and the generic one
    without groups); the smaller ones the 16- and 32-token kernels."""
    g = torch.Generator().manual_seed(77)
    L, T, N = wl.n_layers, wl.T, wl.N
    levels = torch.tensor([0.125, 0.25, 0.5, 0.75])
    s32 = levels[torch.randint(0, 4, (L, T, N), generator=g)].numpy().astype(np.float32)
    bias = None
    if wl.bias_range:  # a bias on a coarse grid keeps keys tied
        bias = (torch.randint(-2, 3, (L, N), generator=g).float() * 0.125)
    out = moer.route(scores=torch.from_numpy(s32).to(DEV), K=wl.K, score_fn=wl.score_fn,
                     n_groups=wl.n_groups, topk_groups=wl.topk_groups, n_shared=wl.n_shared,
                     bias=None if bias is None else bias.to(DEV))
    torch.cuda.synchronize()
    for l in range(L):
        ref = oracle.route(s32=s32[l], bias=None if bias is None else bias[l].numpy(), K=wl.K,
                           score_fn=wl.score_fn, n_groups=wl.n_groups,
                           topk_groups=wl.topk_groups, n_shared=wl.n_shared)
        assert (_np(out["topk_idx"][l]) == ref["idx"]).all(), f"layer {l}"
        assert np.allclose(_np(out["topk_w"][l]).astype(np.float64), ref["w"], rtol=1e-6,
                           atol=1e-7)
        _check_layout(out, l, ref["idx"], wl.Nb)


def test_indices_mode_forcible_balance_and_invalid_ids():
    # MindIE's forcible balancing: supplied ids (t*K + k) mod N -> perfectly even load
    T, K, N = 1000, 8, 256
    t = torch.arange(T)[:, None] * K + torch.arange(K)[None, :]
    idx = (t % N).int()
    out = moer.route(idx_in=idx.to(DEV), K=K, N=N)
    counts = _np(out["counts"][0])
    assert counts.sum() == T * K
    st = moer.decode_load_stats(moer.load_stats(out["counts"], N).cpu())[0]
    ref = oracle.load_stats(counts)
    assert st["imbalance"] == pytest.approx(ref["imbalance"], rel=1e-12)
    _check_layout(out, 0, idx.numpy(), N)
    # repeated and out-of-range ids: kept in slot order / not placed
    idx = torch.tensor([[2, 2], [0, 7], [2, -1]], dtype=torch.int32)
    out = moer.route(idx_in=idx.to(DEV), K=2, N=3)
    assert _np(out["counts"][0]).tolist() == [1, 0, 3]
    assert _np(out["offsets"][0]).tolist() == [0, 1, 1, 4]
    assert _np(out["perm"][0]).tolist() == [2, 0, 1, 4, -1, -1]
    assert _np(out["inv_perm"][0]).tolist() == [1, 2, 0, -1, 3, -1]
    # random ids with shared buckets, several layers
    idx = workloads.make_indices(300, 9, 257, seed=3, n_layers=2)
    out = moer.route(idx_in=idx.to(DEV), K=8, N=256, n_shared=1)
    for l in range(2):
        _check_layout(out, l, idx[l].numpy(), 257)


def _outputs(L, T, N, Kt, Nb):
    i32, f32 = dict(dtype=torch.int32, device=DEV), dict(dtype=torch.float32, device=DEV)
    return dict(topk_idx=torch.empty(L, T, Kt, **i32), topk_w=torch.empty(L, T, Kt, **f32),
                tok_entropy=torch.empty(L, T, **f32), agg_entropy=torch.empty(L, **f32),
                counts=torch.empty(L, Nb, **i32), offsets=torch.empty(L, Nb + 1, **i32),
                perm=torch.empty(L, T * Kt, **i32), inv_perm=torch.empty(L, T * Kt, **i32))


@pytest.mark.parametrize("mode", ["scores", "hidden"])
def test_deterministic_with_poisoned_outputs(mode):
    wl = WL["dsv3_group"] if mode == "scores" else workloads.scaled(WL["dsv3_group"], T=2048)
    b = workloads.make_bias(wl.N, 56).to(DEV)
    if mode == "scores":
        logits = workloads.make_logits(wl.T, wl.N, 55)
        src = dict(scores=torch.from_numpy(_oracle_scores(logits[0], wl.score_fn))[None].to(DEV))
        kind, d = moer.MOER_IN_SCORES, 0
    else:
        inp = workloads.make_inputs(wl)
        src = dict(x=inp["x"].to(DEV), w_gate=inp["W"].to(DEV))
        kind, d = moer.MOER_IN_HIDDEN, wl.d
    desc = moer.make_desc(T=wl.T, d=d, N=wl.N, K=wl.K, n_groups=8, topk_groups=4, input=kind)
    runs = []
    for poison in (0x00, 0xFF):
        outs = _outputs(1, wl.T, wl.N, wl.Kt, wl.Nb)
        ws = torch.empty(moer.moer_route_workspace_bytes(desc), dtype=torch.uint8, device=DEV)
        for v in list(outs.values()) + [ws]:
            v.view(torch.uint8).fill_(poison)
        moer.moer_route(desc, workspace=ws, bias=b, **src, **outs)
        torch.cuda.synchronize()
        runs.append({k: v.view(torch.uint8).cpu().clone() for k, v in outs.items()})
    for k in runs[0]:
        assert torch.equal(runs[0][k], runs[1][k]), k


# ---------------------------------------------------- load stats, bias update
def test_load_stats_parity():
    cases = [[16, 16, 16, 16], [40, 8, 8, 8], [64, 0, 0, 0], [0, 0, 0, 0], [0, 5, 0, 5]]
    g = torch.Generator().manual_seed(8)
    cases.append(torch.randint(0, 1000, (256,), generator=g).tolist())
    for c in cases:
        N = len(c)
        counts = torch.tensor([c + [99]], dtype=torch.int32)  # one shared bucket, excluded
        raw = moer.load_stats(counts.to(DEV), N)
        st = moer.decode_load_stats(raw.cpu())[0]
        ref = oracle.load_stats(np.array(c, np.int32))
        for k in ("total", "max_load", "argmax", "capacity"):
            assert st[k] == ref[k], (c, k)
        for k in ("mean", "imbalance", "h_load_bits", "cv"):
            assert st[k] == pytest.approx(ref[k], rel=1e-9, abs=1e-12), (c, k)


def test_bias_update_bit_exact():
    g = torch.Generator().manual_seed(9)
    L, N = 3, 256
    b = ((torch.rand(L, N, generator=g) * 2 - 1) * 0.01).float()
    counts = torch.randint(480, 545, (L, N + 1), generator=g).int()
    counts[1, :N] = 512
    bd = b.to(DEV)
    moer.bias_update(bd, counts.to(DEV), 1e-3)
    got = _np(bd)
    for l in range(L):
        ref = oracle.bias_update(b[l].numpy(), counts[l, :N].numpy(), 1e-3)
        assert (got[l] == ref).all()
    assert (got[1] == b[1].numpy()).all()


def test_fused_stats_and_bias_update():
    """moer_route's fused load statistics and in-place bias update (bias and
    bias_update the same buffer: selection must read the old values) against
    the oracle, over three consecutive training steps of a 2-layer router."""
    wl = workloads.scaled(WL["collapse_balance"], T=700)
    L = 2
    _, b0, off, _ = workloads.make_router(wl)
    b_gpu = b0.repeat(L, 1).contiguous().to(DEV)
    b_gpu[1] *= -1
    b_ref = [b_gpu[l].cpu().numpy().copy() for l in range(L)]
    for step in range(3):
        logits = workloads.make_logits(wl.T, wl.N, 300 + step, n_layers=L) + off
        s32 = np.stack([_oracle_scores(logits[l], wl.score_fn) for l in range(L)])
        out = moer.route(scores=torch.from_numpy(s32).to(DEV), K=wl.K, n_groups=8, topk_groups=4,
                         bias=b_gpu, want_load_stats=True, bias_update=b_gpu,
                         bias_update_u=2e-3)
        torch.cuda.synchronize()
        got = moer.decode_load_stats(out["load_stats"].cpu())
        for l in range(L):
            ref = oracle.route(s32=s32[l], bias=b_ref[l], K=wl.K, score_fn=wl.score_fn,
                               n_groups=8, topk_groups=4)
            assert (_np(out["topk_idx"][l]) == ref["idx"]).all(), (step, l)
            st = oracle.load_stats(ref["counts"][:wl.N])
            for k in ("total", "max_load", "argmax", "capacity"):
                assert got[l][k] == st[k], (step, l, k)
            for k in ("mean", "imbalance", "h_load_bits", "cv"):
                assert got[l][k] == pytest.approx(st[k], rel=1e-9, abs=1e-12), (step, l, k)
            b_ref[l] = oracle.bias_update(b_ref[l], ref["counts"][:wl.N], 2e-3)
            assert (_np(b_gpu[l]) == b_ref[l]).all(), (step, l)


def test_overlapped_steps_match_one_stream():
    """Consecutive training steps with the bias update, run on one stream and
    then alternating two streams (own workspaces) where step i+1's gate GEMM
    overlaps step i and its selection waits for an event after step i
    (ev_select_wait): every step's counts, ids and updated bias must be
    bitwise the same."""
    import ctypes
    wl = workloads.scaled(WL["collapse_balance"], T=2048, d=1024)
    W, b0, off, gen = workloads.make_router(wl)
    xs = [workloads.make_hidden(wl, seed=500 + i).to(DEV) for i in range(6)]
    desc = moer.make_desc(T=wl.T, d=wl.d, N=wl.N, K=wl.K, n_groups=8, topk_groups=4)
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
    hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def run(nstream):
        streams = [torch.cuda.Stream() for _ in range(nstream)]
        wss = [torch.empty(moer.moer_route_workspace_bytes(desc), dtype=torch.uint8, device=DEV)
               for _ in range(nstream)]
        done = []
        for _ in range(nstream):
            e = ctypes.c_void_p()
            assert hip.hipEventCreateWithFlags(ctypes.byref(e), 0x2) == 0
            done.append(e)
        bias = b0.clone().to(DEV)
        outs = _outputs(1, wl.T, wl.N, wl.Kt, wl.Nb)
        snaps = []
        torch.cuda.synchronize()
        for i, x in enumerate(xs):
            k = i % nstream
            with torch.cuda.stream(streams[k]):
                wait = done[(i - 1) % nstream] if (nstream > 1 and i > 0) else None
                moer.moer_route(desc, workspace=wss[k], x=x, w_gate=W.to(DEV), bias=bias,
                                logit_offset=off.to(DEV), bias_update=bias, bias_update_u=1e-3,
                                ev_select_wait=wait, **outs)
                snaps.append((outs["counts"].clone(), outs["topk_idx"].clone(), bias.clone()))
                assert hip.hipEventRecord(done[k], ctypes.c_void_p(streams[k].cuda_stream)) == 0
        torch.cuda.synchronize()
        for e in done:
            hip.hipEventDestroy(e)
        return [[t.cpu() for t in sn] for sn in snaps]

    one, two = run(1), run(2)
    for i, (a, b) in enumerate(zip(one, two)):
        for name, u, v in zip(("counts", "topk_idx", "bias"), a, b):
            assert torch.equal(u, v), f"step {i}: {name}"
    assert not torch.equal(one[0][2], one[-1][2])  # the bias did move


def _lockstep(wl, rounds, b_gpu, b_ref, first=0):
    """Rounds first .. first+rounds-1 of the collapse loop (hotdry,
    auxiliary-loss-free balancing: route -> count -> sign step) on identical
    fp32 scores, GPU and oracle each applying its own update. Returns the
    per-round counts and biases of both sides."""
    off = workloads.make_router(wl)[2]
    hist = []
    for i in range(first, first + rounds):
        logits = workloads.make_logits(wl.T, wl.N, 1000 + i)[0] + off
        s32 = _oracle_scores(logits, wl.score_fn)
        out = moer.route(scores=torch.from_numpy(s32)[None].to(DEV), K=wl.K, n_groups=8,
                         topk_groups=4, bias=b_gpu, want_entropy=False, want_inv_perm=False,
                         bias_update=b_gpu, bias_update_u=1e-3)
        ref = oracle.route(s32=s32, bias=b_ref, K=wl.K, score_fn=wl.score_fn, n_groups=8,
                           topk_groups=4)
        b_ref = oracle.bias_update(b_ref, ref["counts"][:wl.N], 1e-3)
        hist.append((_np(out["counts"][0]), ref["counts"], _np(b_gpu[0]).copy(), b_ref.copy()))
    return hist, b_ref


@pytest.mark.timeout(900)
def test_collapse_balancing_lockstep_full_size():
    """The collapse workload at its own size (16384 tokens, celebrity experts
    with a +3.0 logit offset) for all 100 rounds, GPU and oracle in lockstep
    on identical fp32 scores; the GPU's update is the one fused into the
    route call. Counts and biases must stay bit-identical every round."""
    wl = WL["collapse_balance"]
    _, b0, _, _ = workloads.make_router(wl)
    b_gpu = b0.clone().to(DEV)
    hist, _ = _lockstep(wl, 100, b_gpu, b0[0].numpy().copy())
    imb = []
    for i, (gc, rc, gb, rb) in enumerate(hist):
        assert (gc == rc).all(), f"round {i}: counts"
        assert (gb == rb).all(), f"round {i}: bias"
        imb.append(oracle.load_stats(rc[:wl.N])["imbalance"])
    say("  imbalance every 10 rounds: " + " ".join(f"{v:.2f}" for v in imb[::10]) +
        f" ... {imb[-1]:.2f}")
    assert imb[-1] < imb[0]


def test_collapse_loop_resumes_from_round_and_bias():
    """The loop's whole state is (round i, bias b_i): restarted from a saved
    (i, b_i), both the GPU and the oracle continue with exactly the counts
    and biases of the uninterrupted run."""
    wl = workloads.scaled(WL["collapse_balance"], T=2048)
    _, b0, _, _ = workloads.make_router(wl)
    full, _ = _lockstep(wl, 20, b0.clone().to(DEV), b0[0].numpy().copy())
    saved_gpu, saved_ref = full[9][2], full[9][3]          # after round 9: b_10
    assert (saved_gpu == saved_ref).all()
    resumed, _ = _lockstep(wl, 10, torch.from_numpy(saved_gpu.copy())[None].to(DEV),
                           saved_ref.copy(), first=10)
    for k, (a, b) in enumerate(zip(full[10:], resumed)):
        for j, name in enumerate(("gpu counts", "oracle counts", "gpu bias", "oracle bias")):
            assert (a[j] == b[j]).all(), f"round {10 + k}: {name}"


@pytest.mark.timeout(900)
@pytest.mark.parametrize("T,d,batches", [(1024, 1024, 30), (16384, 7168, 10)],
                         ids=["small-30", "full-10"])
def test_collapse_free_running_hidden_mode(T, d, batches):
    """The collapse loop in HIDDEN mode, GPU and oracle each running free
    (each updates its own bias from its own counts), at a small size for 30
    batches and at the workload's own size (16384 tokens, d = 7168) for 10.
    Every batch, the GPU's decisions are checked against the oracle run with
    the GPU's current bias (a token may differ only under the near-tie rule,
    and the count differences are exactly those tokens'), and the GPU's bias
    update against the oracle's update of the GPU's counts (bit-exact). Both
    trajectories are reported."""
    wl = workloads.scaled(WL["collapse_balance"], T=T, d=d)
    W, b0, off, _ = workloads.make_router(wl)
    Wd, offd = W.to(DEV), off.to(DEV)
    b_gpu = b0.clone().to(DEV)
    b_free = b0[0].numpy().copy()
    kw = dict(K=wl.K, score_fn=wl.score_fn, n_groups=wl.n_groups, topk_groups=wl.topk_groups)
    traj_gpu, traj_free, near = [], [], 0
    for i in range(batches):
        x = workloads.make_hidden(wl, seed=1000 + i)
        b_before = _np(b_gpu[0]).copy()
        out = moer.route(x.to(DEV), Wd, bias=b_gpu, logit_offset=offd, bias_update=b_gpu,
                         bias_update_u=1e-3, want_entropy=False, **kw)
        torch.cuda.synchronize()
        xs, Ws = x[0].float().numpy(), W[0].float().numpy()
        shadow = oracle.route(x=xs, W=Ws, offset=off.numpy(), bias=b_before, **kw)
        gi = _np(out["topk_idx"][0])
        diff = ~(gi == shadow["idx"]).all(axis=1)
        assert np.all(~diff | (shadow["gap"] < 1e-3)), f"batch {i}: beyond the near-tie rule"
        near += int(diff.sum())
        gc = _np(out["counts"][0])[:wl.N]
        expect = shadow["counts"][:wl.N].astype(np.int64)
        for t in np.nonzero(diff)[0]:
            np.add.at(expect, gi[t], 1)
            np.add.at(expect, shadow["idx"][t], -1)
        assert (gc == expect).all(), f"batch {i}: counts not explained by near ties"
        assert (_np(b_gpu[0]) == oracle.bias_update(b_before, gc, 1e-3)).all(), f"batch {i}"
        free = oracle.route(x=xs, W=Ws, offset=off.numpy(), bias=b_free, **kw)
        b_free = oracle.bias_update(b_free, free["counts"][:wl.N], 1e-3)
        traj_gpu.append(oracle.load_stats(gc)["imbalance"])
        traj_free.append(oracle.load_stats(free["counts"][:wl.N])["imbalance"])
    say(f"  {batches} batches of {T} tokens, near-tie differences {near}")
    say("  imbalance, GPU free-running:    " + " ".join(f"{v:.2f}" for v in traj_gpu[::5]))
    say("  imbalance, oracle free-running: " + " ".join(f"{v:.2f}" for v in traj_free[::5]))
    assert traj_gpu[-1] < traj_gpu[0] and traj_free[-1] < traj_free[0]


# ------------------------------------------- balancing-rule variants
@pytest.mark.parametrize("wl", [
    workloads.scaled(WL["mixtral_top2"], T=600),
    workloads.scaled(WL["dsv3_group"], T=500),
    workloads.scaled(WL["collapse_balance"], T=300),
    workloads.scaled(WL["decode_layers"], n_layers=3, T=70),
], ids=lambda w: f"{w.name}-T{w.T}-L{w.n_layers}")
def test_logit_space_bias_hidden_mode(wl):
    # The dailyaiworld controller's reading: the bias joins the logits, and
    # scores, selection, weights and entropy all come from h + b. A bias of
    # +-0.5 (larger than the score-space one) makes the shift visible.
    say(f"[logit bias] {wl}")
    g = torch.Generator().manual_seed(31)
    b = ((torch.rand(wl.n_layers, wl.N, generator=g) * 2 - 1) * 0.5).float()
    _hidden_case(wl, wl.name + "/logit", bias_mode="logit", bias=b)


BALANCE_CFGS = [
    dict(rule="sign", step=1e-3, alpha=1.0, every=1),
    dict(rule="proportional", step=0.05, alpha=1.0, every=1),
    dict(rule="sign", step=2e-3, alpha=0.25, every=3),
    dict(rule="proportional", step=0.05, alpha=0.1, every=2),
]


@pytest.mark.parametrize("cfg", BALANCE_CFGS, ids=lambda c: "-".join(str(v) for v in c.values()))
@pytest.mark.parametrize("L,N,stride", [(3, 256, 256), (2, 8, 8), (4, 256, 257)])
def test_balance_step_bit_exact_over_calls(cfg, L, N, stride):
    say(f"[balance step] {cfg} L={L} N={N}")
    g = np.random.default_rng(N + L)
    b0 = g.uniform(-0.01, 0.01, (L, N)).astype(np.float32)
    bias = torch.from_numpy(b0).to(DEV)
    state = moer.BalanceState(L, N)
    ref = [dict(b=b0[l].copy(), loads=np.zeros(N, np.float32), calls=0) for l in range(L)]
    for call in range(7):
        counts = g.integers(0, 900, (L, stride)).astype(np.int32)
        if call == 4:
            counts[:, :N] = 512   # a balanced call: the rules leave the bias alone
        moer.balance_step(bias, torch.from_numpy(counts).to(DEV), state=state, **cfg)
        torch.cuda.synchronize()
        for l in range(L):
            r = ref[l]
            r["b"], r["loads"], r["calls"] = oracle.balance_step(
                r["b"], counts[l, :N], rule=oracle.SIGN if cfg["rule"] == "sign" else
                oracle.PROPORTIONAL, step=cfg["step"], alpha=cfg["alpha"], every=cfg["every"],
                loads=r["loads"], calls=r["calls"])
            assert (_np(bias[l]) == r["b"]).all(), f"call {call} layer {l}: bias"
            assert (_np(state.loads[l]) == r["loads"]).all(), f"call {call} layer {l}: loads"
            assert int(state.calls[l]) == r["calls"]


def test_balance_step_sign_equals_bias_update():
    g = np.random.default_rng(5)
    counts = torch.from_numpy(g.integers(300, 700, (2, 257)).astype(np.int32)).to(DEV)
    b = torch.from_numpy(g.uniform(-0.01, 0.01, (2, 256)).astype(np.float32)).to(DEV)
    a, c = b.clone(), b.clone()
    moer.balance_step(a, counts, rule="sign", step=1e-3)
    moer.bias_update(c, counts, 1e-3)
    torch.cuda.synchronize()
    assert torch.equal(a, c)


def test_dailyaiworld_controller_loop():
    # The listing's controller run for 12 batches on the collapse workload
    # (celebrity experts): logit-space bias, proportional update with decay
    # 0.05. Each step is checked against the oracle on the GPU's own counts
    # (selections within the near-tie rule); the celebrities' bias must fall.
    wl = workloads.scaled(WL["collapse_balance"], T=1024, d=1024)
    say(f"[controller] {wl}")
    W, b0, off, _ = workloads.make_router(wl)
    bias = torch.zeros(1, wl.N, device=DEV)
    b_ref = np.zeros(wl.N, np.float32)
    for it in range(12):
        x = workloads.make_hidden(wl, seed=2000 + it)
        out = moer.route(x.to(DEV), W.to(DEV), K=wl.K, n_groups=wl.n_groups,
                         topk_groups=wl.topk_groups, bias=bias, logit_offset=off.to(DEV),
                         bias_mode="logit", want_h=True)
        torch.cuda.synchronize()
        ref = oracle.route(x=x[0].float().numpy(), W=W[0].float().numpy(), offset=off.numpy(),
                           bias=b_ref, K=wl.K, score_fn=wl.score_fn, n_groups=wl.n_groups,
                           topk_groups=wl.topk_groups, bias_mode="logit")
        gi = _np(out["topk_idx"][0])
        same = (gi == ref["idx"]).all(axis=1)
        assert np.all(same | (ref["gap"] < 1e-3)), f"batch {it}"
        counts = out["counts"]
        moer.balance_step(bias, counts, rule="proportional", step=0.05)
        torch.cuda.synchronize()
        b_ref, _, _ = oracle.balance_step(b_ref, _np(counts[0])[:wl.N], rule=oracle.PROPORTIONAL,
                                          step=0.05)
        assert (_np(bias[0]) == b_ref).all(), f"batch {it}: bias"
    celeb = list(wl.celebrities)
    assert (b_ref[celeb] < 0).all()


# ---------------------------------------------------------------------------
# Seeded random router shapes: expert counts, group geometries, K, shared
# slots, token counts around the 32/64-token block edges, layers, score
# functions and bias scales that the fixed cases above do not cover. A shape
# these kernels refuse as unsupported (MOER_EUNSUPPORTED: a group width the
# row kernels cannot split) is skipped; everything else must meet the
# SCORES-mode (bit-exact) or HIDDEN-mode bars.

def _random_router(i, hidden=False):
    rng = np.random.default_rng(1000 + i)
    N = int(rng.choice([1, 2, 3, 4, 7, 8, 16, 24, 32, 60, 64, 100, 128, 160, 200, 255, 256]))
    divs = [g for g in range(1, N + 1) if N % g == 0 and (g == 1 or N // g >= 2)]
    G = int(rng.choice(divs))
    Gk = int(rng.integers(1, G + 1))
    K = int(rng.integers(1, min(Gk * (N // G), 16) + 1))
    n_shared = int(rng.integers(0, 16 - K + 1)) if rng.random() < 0.3 else 0
    L = int(rng.choice([1, 1, 2, 3]))
    T = int(rng.choice([1, 2, 31, 32, 33, 63, 64, 65, 127, 128, 129, 500, 1000, 2047, 2048,
                        2049, 3001]))
    score_fn = workloads.SIGMOID if rng.random() < 0.5 else workloads.SOFTMAX
    bias_range = float(rng.choice([0.0, 0.01, 0.3]))
    d = int(rng.choice([8, 40, 64, 72, 136, 264, 520, 1024])) if hidden else 64
    dtype = workloads.F32 if hidden and rng.random() < 0.3 else workloads.BF16
    if hidden:
        T = min(T, 1000)
    return workloads.Workload(f"random{i}", T=T, d=d, N=N, K=K, score_fn=score_fn, dtype=dtype,
                              n_groups=G, topk_groups=Gk, n_shared=n_shared, n_layers=L,
                              bias_range=bias_range, seed=2000 + i)


def _run_or_skip(fn, wl):
    try:
        return fn()
    except moer.MoerError as exc:
        if exc.status == moer.MOER_EUNSUPPORTED:
            pytest.skip(f"unsupported shape {wl}: {exc}")
        raise


@pytest.mark.parametrize("i", range(120))
def test_scores_mode_bit_exact_random_shapes(i):
    wl = _random_router(i)
    say(f"[scores/random {i}] {wl}")
    _run_or_skip(lambda: _scores_case(wl, seed=3000 + i), wl)


@pytest.mark.parametrize("i", range(30))
def test_hidden_mode_random_shapes(i):
    wl = _random_router(i, hidden=True)
    say(f"[hidden/random {i}] {wl}")
    _run_or_skip(lambda: _hidden_case(wl, wl.name), wl)


# ---------------------------------------------------------------------------
# Non-finite inputs: the results are unspecified, but every id stays in range
# and the layout stays a consistent stable permutation of the ids produced.

def _check_consistent(out, wl):
    for l in range(wl.n_layers):
        gi = _np(out["topk_idx"][l])
        routed, shared = gi[:, :wl.K], gi[:, wl.K:]
        assert ((routed >= -1) & (routed < wl.N)).all()
        assert (shared == wl.N + np.arange(wl.n_shared)).all()
        ids = np.where(gi >= 0, gi, -1)
        if (ids < 0).any():  # capacity drops: the layout skips them
            valid = ids[ids >= 0]
            assert _np(out["counts"][l]).sum() == valid.size
            continue
        _check_layout(out, l, ids, wl.Nb)


@pytest.mark.parametrize("capacity", [0, 1])
@pytest.mark.parametrize("wl", [
    workloads.scaled(WL["dsv3_group"], T=700),
    workloads.scaled(WL["decode_layers"], n_layers=2, T=130),
    workloads.scaled(WL["dsv3_group"], T=200, N=96, n_groups=8, topk_groups=4, K=6),
    WL["dsv3_group"],
], ids=lambda w: f"{w.name}-T{w.T}-N{w.N}")
def test_non_finite_scores_stay_in_range(wl, capacity):
    say(f"[non-finite scores] {wl} capacity={capacity}")
    rng = np.random.default_rng(5)
    s = rng.random((wl.n_layers, wl.T, wl.N)).astype(np.float32)
    mask = rng.random(s.shape)
    s[mask < 0.02] = np.nan
    s[(mask >= 0.02) & (mask < 0.04)] = np.inf
    s[(mask >= 0.04) & (mask < 0.05)] = -np.inf
    s[0, :3] = np.nan  # whole rows of NaN
    cap = moer.expert_capacity(wl.T, wl.K, wl.N) if capacity else 0
    out = moer.route(scores=torch.from_numpy(s).to(DEV), K=wl.K, score_fn=wl.score_fn,
                     n_groups=wl.n_groups, topk_groups=wl.topk_groups, n_shared=wl.n_shared,
                     capacity=cap)
    torch.cuda.synchronize()
    _check_consistent(out, wl)
    if cap:
        assert _np(out["counts"])[:, :wl.N].max() <= cap


# Hidden-state paths: the 256-expert GEMM + selection; the one-launch kernel
# of routers with at most 16 experts (16-token workgroups); the one-workgroup
# layer kernel in rows of 8, 4 and 16 lanes (the last one grouped, with
# shared slots).
SMALL_PATHS = [
    workloads.scaled(WL["dsv3_group"], T=300, d=512),
    workloads.scaled(WL["mixtral_top2"], T=300, d=512),
    workloads.scaled(WL["mixtral_top2"], T=40, d=256),
    WL["tiny_softmax"],
    workloads.scaled(WL["mixtral_top2"], T=24, d=256, N=16, K=4, n_groups=4, topk_groups=2,
                     n_shared=2),
]


@pytest.mark.parametrize("wl", SMALL_PATHS,
                         ids=lambda w: f"{w.name}-T{w.T}-d{w.d}-N{w.N}-G{w.n_groups}")
def test_non_finite_hidden_states_stay_in_range(wl):
    say(f"[non-finite hidden] {wl}")
    inp = workloads.make_inputs(wl)
    x = inp["x"].clone()
    x[0, 5, 7] = float("inf")
    x[0, 9, :] = float("nan")
    x[0, 11, 3] = -float("inf")
    out = moer.route(x.to(DEV), inp["W"].to(DEV), K=wl.K, score_fn=wl.score_fn,
                     n_groups=wl.n_groups, topk_groups=wl.topk_groups, n_shared=wl.n_shared,
                     bias=inp["bias"].to(DEV), want_h=True, want_load_stats=True)
    torch.cuda.synchronize()
    _check_consistent(out, wl)
    # the rows without a non-finite element route as they do without the others
    clean = moer.route(inp["x"].to(DEV), inp["W"].to(DEV), K=wl.K, score_fn=wl.score_fn,
                       n_groups=wl.n_groups, topk_groups=wl.topk_groups, n_shared=wl.n_shared,
                       bias=inp["bias"].to(DEV), want_h=True)
    torch.cuda.synchronize()
    keep = np.ones(wl.T, dtype=bool)
    keep[[5, 9, 11]] = False
    for k in ("h", "topk_idx", "topk_w", "tok_entropy"):
        assert torch.equal(out[k][0].cpu()[keep], clean[k][0].cpu()[keep]), k


@pytest.mark.parametrize("wl", SMALL_PATHS[1:],
                         ids=lambda w: f"{w.name}-T{w.T}-d{w.d}-N{w.N}-G{w.n_groups}")
def test_hidden_mode_small_routers_workspace_contents_do_not_matter(wl):
    # the one-launch small-router kernels and their layout take the caller's
    # workspace as scratch too: zero-filled and random bytes give the same bits
    say(f"[small-router workspace] {wl}")
    inp = workloads.make_inputs(wl)
    off = None if inp["offset"] is None else inp["offset"].to(DEV)
    gen = torch.Generator(device="cpu").manual_seed(11)
    runs = []
    for fill in ("zeros", "random"):
        ws = torch.zeros(16 << 20, dtype=torch.uint8, device=DEV)  # ample for these shapes
        if fill == "random":
            ws.copy_(torch.randint(0, 256, (ws.numel(),), dtype=torch.uint8, generator=gen))
        bias = inp["bias"].float().to(DEV)
        out = moer.route(inp["x"].to(DEV), inp["W"].to(DEV), K=wl.K, score_fn=wl.score_fn,
                         n_groups=wl.n_groups, topk_groups=wl.topk_groups,
                         n_shared=wl.n_shared, bias=bias, logit_offset=off, want_h=True,
                         want_load_stats=True, bias_update=bias, workspace=ws)
        torch.cuda.synchronize()
        runs.append({k: v.cpu().clone() for k, v in out.items() if torch.is_tensor(v)})
        runs[-1]["bias"] = bias.cpu()
    for k in runs[0]:
        assert torch.equal(runs[0][k], runs[1][k]), f"{k} depends on the workspace"


@pytest.mark.parametrize("case", ["capacity", "indices", "decode_layers", "any_groups"])
def test_workspace_contents_do_not_matter(case):
    # the caller's workspace may hold anything: a zero-filled one and one of
    # random bytes give bitwise-identical outputs
    if case == "decode_layers":
        wl = workloads.scaled(WL["decode_layers"], n_layers=5, T=100)
    elif case == "any_groups":
        wl = workloads.scaled(WL["dsv3_group"], T=500, N=96, n_groups=8, topk_groups=4, K=6)
    else:
        wl = workloads.scaled(WL["dsv3_group"], T=900)
    L = wl.n_layers
    logits = workloads.make_logits(wl.T, wl.N, 77, n_layers=L).double().numpy()
    logits[..., :4] += 3.0  # a few experts over capacity
    s32 = np.stack([oracle.scores(logits[l], wl.score_fn).astype(np.float32) for l in range(L)])
    kw = dict(K=wl.K, score_fn=wl.score_fn, n_groups=wl.n_groups, topk_groups=wl.topk_groups,
              n_shared=wl.n_shared, want_load_stats=True)
    if case == "indices":
        ids = torch.from_numpy(np.stack([oracle.route(s32=s32[l], K=wl.K, score_fn=wl.score_fn,
                                                      n_groups=wl.n_groups,
                                                      topk_groups=wl.topk_groups)["idx"]
                                         for l in range(L)]).astype(np.int32))
        kw = dict(K=wl.K, N=wl.N, idx_in=ids.to(DEV), want_load_stats=True)
    else:
        kw["scores"] = torch.from_numpy(s32).to(DEV)
        if case == "capacity":
            kw["capacity"] = moer.expert_capacity(wl.T, wl.K, wl.N)
    runs = []
    gen = torch.Generator(device="cpu").manual_seed(9)
    for fill in ("zeros", "random"):
        ws = torch.zeros(64 << 20, dtype=torch.uint8, device=DEV)  # ample for these shapes
        if fill == "random":
            ws.copy_(torch.randint(0, 256, (ws.numel(),), dtype=torch.uint8, generator=gen))
        out = moer.route(workspace=ws, **kw)
        torch.cuda.synchronize()
        runs.append({k: v.cpu().clone() for k, v in out.items() if torch.is_tensor(v)})
    for k in runs[0]:
        assert torch.equal(runs[0][k], runs[1][k]), f"{case}: {k} depends on the workspace"
