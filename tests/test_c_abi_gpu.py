"""The router's C ABI driven from a plain C program (GPU).

tests/c_abi/moer_route_c is a C11 program that uses only include/moer.h and
the HIP runtime's C API (built by build() with gcc). It runs moer_route with
the load statistics fused in, then the standalone moer_load_stats and
moer_bias_update on the counts, and writes every output to a file. Here its
outputs are held to two bars on the same seeded inputs:
- bit for bit equal to the Python binding's call of the same library, whose
  bias update is the one fused into moer_route. That equality shows the
  standalone statistics and the standalone sign step give the fused ones'
  bits;
- against the CPU oracle: selections by the near-tie rule, weights within
  1e-3, entropies within 1e-4 bits, the layout of the program's own ids
  exactly, the load statistics (integers exact, derived values 1e-9
  relative) and the bias update exactly.
The shapes cover the one-workgroup layer kernel (fp32 toy router), the
16-token small-router kernel, the DeepSeek-V3 group-limited path, and two
decode-shaped layers with a shared slot. The toy router's case also times
200 back-to-back calls from C and reports them (no bar).
"""
import os
import struct
import subprocess

import numpy as np
import pytest
import torch

import oracle
import top_expert_routing_gate_amd as moer
import workloads

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
WL = workloads.WORKLOADS
EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "moer_route_c")
MAGIC = 0x524F454D
U = 1e-3
SCORE_FN = {workloads.SOFTMAX: moer.MOER_SOFTMAX, workloads.SIGMOID: moer.MOER_SIGMOID}

CASES = [
    (WL["tiny_softmax"], 200),
    (workloads.scaled(WL["mixtral_top2"], T=300, d=512), 0),
    (workloads.scaled(WL["dsv3_group"], T=500, d=1024), 0),
    (workloads.scaled(WL["decode_layers"], n_layers=2, T=70, d=512), 0),
]


def say(msg):
    print(msg, flush=True)


def _raw(t):
    t = t.contiguous()
    return (t.view(torch.int16) if t.dtype == torch.bfloat16 else t).numpy().tobytes()


def _write_input(path, wl, inp, timed):
    dtype = moer.MOER_BF16 if inp["x"].dtype == torch.bfloat16 else moer.MOER_F32
    hdr = struct.pack("<12i", MAGIC, wl.n_layers, wl.T, wl.d, wl.N, wl.K, wl.n_groups,
                      wl.topk_groups, wl.n_shared, SCORE_FN[wl.score_fn], dtype, timed)
    with open(path, "wb") as f:
        f.write(hdr + struct.pack("<f", U) + _raw(inp["x"]) + _raw(inp["W"]) +
                _raw(inp["bias"].float()))


def _read_output(path, wl):
    L, T, Kt, Nb, N = wl.n_layers, wl.T, wl.Kt, wl.Nb, wl.N
    b = open(path, "rb").read()
    out, pos = {}, 0

    def take(name, dtype, shape):
        nonlocal pos
        n = int(np.prod(shape)) * np.dtype(dtype).itemsize
        out[name] = np.frombuffer(b[pos:pos + n], dtype=dtype).reshape(shape)
        pos += n

    take("topk_idx", np.int32, (L, T, Kt))
    take("topk_w", np.float32, (L, T, Kt))
    take("tok_entropy", np.float32, (L, T))
    take("agg_entropy", np.float32, (L,))
    take("counts", np.int32, (L, Nb))
    take("offsets", np.int32, (L, Nb + 1))
    take("perm", np.int32, (L, T * Kt))
    take("inv_perm", np.int32, (L, T * Kt))
    take("stats_fused", np.uint8, (L, 64))
    take("stats", np.uint8, (L, 64))
    take("bias", np.float32, (L, N))
    take("timing", np.float32, (2,))
    assert pos == len(b), "unexpected output size"
    return out


@pytest.mark.parametrize("wl,timed", CASES,
                         ids=lambda c: f"{c.name}-T{c.T}-L{c.n_layers}" if hasattr(c, "name")
                         else f"timed{c}")
def test_c_program_matches_binding_and_oracle(wl, timed, tmp_path):
    if not os.path.exists(EXE):
        pytest.skip("the C driver is not built (run __graft_entry__.build())")
    say(f"[C ABI] {wl}")
    inp = workloads.make_inputs(wl)
    fin, fout = str(tmp_path / "in.bin"), str(tmp_path / "out.bin")
    _write_input(fin, wl, inp, timed)
    r = subprocess.run([EXE, fin, fout], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"C driver failed ({r.returncode}):\n{r.stdout}\n{r.stderr}"
    got = _read_output(fout, wl)
    if timed:
        say(f"  from C: {r.stdout.strip()}")
        assert got["timing"][0] > 0 and got["timing"][1] > 0

    # the Python binding, same library, fused statistics and bias update
    bias = inp["bias"].float().to(DEV)
    ref = moer.route(inp["x"].to(DEV), inp["W"].to(DEV), K=wl.K, score_fn=wl.score_fn,
                     n_groups=wl.n_groups, topk_groups=wl.topk_groups, n_shared=wl.n_shared,
                     bias=bias, want_load_stats=True, bias_update=bias, bias_update_u=U)
    torch.cuda.synchronize()
    for k in ("topk_idx", "topk_w", "tok_entropy", "agg_entropy", "counts", "offsets", "perm",
              "inv_perm"):
        assert np.array_equal(got[k], ref[k].cpu().numpy()), f"{k} differs from the binding"
    raw = ref["load_stats"].cpu().numpy()
    assert np.array_equal(got["stats_fused"], raw), "fused statistics differ"
    assert np.array_equal(got["stats"], raw), "moer_load_stats differs from the fused records"
    assert np.array_equal(got["bias"], bias.cpu().numpy()), "moer_bias_update differs"

    # the oracle
    stats = moer.decode_load_stats(torch.from_numpy(got["stats"].copy()))
    x, W = inp["x"].float().numpy(), inp["W"].float().numpy()
    for l in range(wl.n_layers):
        b0 = inp["bias"][l].float().numpy()
        o = oracle.route(x=x[l], W=W[l], bias=b0, K=wl.K, score_fn=wl.score_fn,
                         n_groups=wl.n_groups, topk_groups=wl.topk_groups,
                         n_shared=wl.n_shared)
        gi = got["topk_idx"][l]
        same = (gi == o["idx"]).all(axis=1)
        assert np.all(same | (o["gap"] < 1e-3)), "selection differs beyond the near-tie rule"
        assert np.abs(got["topk_w"][l][same] - o["w"][same]).max() < 1e-3
        assert np.abs(got["tok_entropy"][l] - o["tok_H"]).max() < 1e-4
        assert abs(float(got["agg_entropy"][l]) - o["agg_H"]) < 1e-4
        counts, offsets, perm, inv = oracle.layout(gi, wl.Nb)
        assert (got["counts"][l] == counts).all() and (got["offsets"][l] == offsets).all()
        assert (got["perm"][l] == perm).all() and (got["inv_perm"][l] == inv).all()
        st = oracle.load_stats(counts[:wl.N])
        for k in ("total", "max_load", "argmax", "capacity"):
            assert stats[l][k] == st[k], k
        for k in ("mean", "imbalance", "h_load_bits", "cv"):
            assert stats[l][k] == pytest.approx(st[k], rel=1e-9, abs=1e-12), k
        nb = oracle.bias_update(b0.copy(), counts[:wl.N], U)
        assert (got["bias"][l] == nb).all(), "bias update differs from the oracle's"
