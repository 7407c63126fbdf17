"""The oracle's pins must catch plausible mistakes (CPU only).

Each mutant below plants one slip in a copy of oracle/moero.c — a flipped
sign, a dropped term, a wrong index, tie-break or normalisation — builds it,
and runs the pin suite (tests/test_oracle_pins.py) against that build. Every
mutant must make at least one pin fail; a surviving mutant means the pins
leave that part of the oracle unchecked.
"""
import concurrent.futures
import os
import subprocess
import sys
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "moero.c")

MUTANTS = [
    ("affinity operand index", "acc += (double)xt[k] * (double)we[k];",
     "acc += (double)xt[k] * (double)we[(k + 1) % d];"),
    ("logit offset sign", "if (offset) acc += (double)offset[e];",
     "if (offset) acc -= (double)offset[e];"),
    ("sigmoid sign", "st[e] = 1.0 / (1.0 + exp(-ht[e]));", "st[e] = 1.0 / (1.0 + exp(ht[e]));"),
    ("softmax normaliser", "for (int32_t e = 0; e < N; ++e) st[e] /= z;",
     "for (int32_t e = 0; e < N; ++e) st[e] /= (z + 1.0);"),
    ("bias sign", "volatile float k = st[e] + (bias ? bias[e] : 0.0f);",
     "volatile float k = st[e] - (bias ? bias[e] : 0.0f);"),
    ("group score = top-1 only", "volatile float gs = mem[0].v + mem[1].v;",
     "volatile float gs = mem[0].v;"),
    ("id tie-break reversed", "return (a->id > b->id) - (a->id < b->id);",
     "return (a->id < b->id) - (a->id > b->id);"),
    ("kept groups off by one", "for (int32_t r = 0; r < Gk; ++r) kept[grp[r].id] = 1;",
     "for (int32_t r = 1; r <= Gk && r < G; ++r) kept[grp[r].id] = 1;"),
    ("weights from biased keys", "for (int32_t k = 0; k < K; ++k) z += sd[cand[k].id];",
     "for (int32_t k = 0; k < K; ++k) z += cand[k].v;"),
    ("shared slot weight", "w[(size_t)t * Kt + K + j] = 1.0f;\n        }\n        /* 6.",
     "w[(size_t)t * Kt + K + j] = 0.0f;\n        }\n        /* 6."),
    ("entropy in nats", "if (q > 0.0) H -= q * log2(q);", "if (q > 0.0) H -= q * log(q);"),
    ("aggregate of unnormalised scores", "mean[e] += sd[e] / z;", "mean[e] += sd[e];"),
    ("layout order within an expert",
     "for (int64_t a = 0; a < A; ++a) {\n      if (idx[a] == e) {",
     "for (int64_t a = A - 1; a >= 0; --a) {\n      if (idx[a] == e) {"),
    ("offsets inclusive", "offsets[e + 1] = offsets[e] + counts[e];",
     "offsets[e + 1] = offsets[e] + counts[e] + (e == 0 ? counts[0] : 0);"),
    ("capacity formula", "out->capacity = mx * (int64_t)N;", "out->capacity = mx + (int64_t)N;"),
    ("imbalance over total", "out->imbalance = out->mean != 0.0 ? (double)mx / out->mean : 0.0;",
     "out->imbalance = out->mean != 0.0 ? (double)mx / (double)total : 0.0;"),
    ("argmax tie to the highest id", "if (counts[e] > mx) { mx = counts[e]; am = e; }",
     "if (counts[e] >= mx) { mx = counts[e]; am = e; }"),
    ("sample instead of population std", "var = N > 0 ? var / (double)N : 0.0;",
     "var = N > 1 ? var / (double)(N - 1) : 0.0;"),
    ("bias update sign", "float step = diff > 0 ? u : (diff < 0 ? -u : 0.0f);",
     "float step = diff > 0 ? -u : (diff < 0 ? u : 0.0f);"),
    ("bias update ignores balance", "float step = diff > 0 ? u : (diff < 0 ? -u : 0.0f);",
     "float step = diff >= 0 ? u : -u;"),
    ("gap misses the top-K boundary",
     "double dk = (double)cand[K - 1].v - (double)cand[K].v;\n          if (dk < margin) margin = dk;",
     "double dk = (double)cand[K - 1].v - (double)cand[K].v;\n          (void)dk;"),
    ("dispatch token from the slot index", "const int64_t t = perm[pos] / Kt;",
     "const int64_t t = perm[pos] % Kt;"),
    ("dispatch drops the first slot", "if (perm[pos] < 0) continue;", "if (perm[pos] <= 0) continue;"),
    ("combine weight of the token's first slot", "const double wk = (double)w[slot];",
     "const double wk = (double)w[t * Kt];"),
    ("combine keeps only the last slot", "y[t * d + j] += wk * out[pos * d + j];",
     "y[t * d + j] = wk * out[pos * d + j];"),
    ("combine skips position 0",
     "for (int64_t pos = 0; pos < A; ++pos) {\n    const int32_t slot = perm[pos];",
     "for (int64_t pos = 1; pos < A; ++pos) {\n    const int32_t slot = perm[pos];"),
    ("balanced ids restart per token", "idx[(int64_t)t * Kt + k] = (int32_t)(((int64_t)t * K + k + start) % N);",
     "idx[(int64_t)t * Kt + k] = (int32_t)(((int64_t)k + start) % N);"),
    ("balanced ids ignore the start", "int64_t start = first % N;", "int64_t start = 0 * first;"),
    ("hotspot reads the wrong stride",
     "hot[(int64_t)l * N + e] += counts[(int64_t)l * stride + e];",
     "hot[(int64_t)l * N + e] += counts[(int64_t)l * N + e];"),
    ("logit bias subtracted", "h[(int64_t)t * N + e] += (double)b[e];",
     "h[(int64_t)t * N + e] -= (double)b[e];"),
    ("moving average weights swapped", "volatile float fresh = alpha * ce;",
     "volatile float fresh = keep * ce;"),
    ("proportional rule sign", "volatile float nb = bias[e] - delta;",
     "volatile float nb = bias[e] + delta;"),
    ("proportional error over N", "const double rel = ((double)l[e] - mean) / mean;",
     "const double rel = ((double)l[e] - mean) / (double)N;"),
    ("period off by one", "if ((ncall + 1) % every == 0) {", "if (ncall % every == 0) {"),
    ("sign rule against the total", "const double diff = mean - (double)l[e];",
     "const double diff = total - (double)l[e];"),
    ("capacity admits one more", "if (held[e] < cap) { held[e] += 1; state[a] = ACCEPTED; }",
     "if (held[e] <= cap) { held[e] += 1; state[a] = ACCEPTED; }"),
    ("capacity accepts latest tokens first",
     "for (int64_t a = 0; a < A; ++a) {\n      if (state[a] != PENDING) continue;",
     "for (int64_t a = A - 1; a >= 0; --a) {\n      if (state[a] != PENDING) continue;"),
    ("rejected slots skip a candidate", "prop[a] = list[(size_t)t * N + next[t]];\n        next[t] += 1;",
     "next[t] += 1;\n        prop[a] = list[(size_t)t * N + (next[t] < n_el[t] ? next[t] : next[t] - 1)];"),
    ("dropped slots keep a weight", "w[(size_t)t * Kt + k] = dropped_slot ? 0.0f",
     "w[(size_t)t * Kt + k] = dropped_slot ? 1.0f"),
    ("reroute count of every placed slot", "if (prop[a] != list[(size_t)t * N + k]) ++rerouted;",
     "++rerouted;"),
]


def _build(src_text, out_dir, name):
    c = os.path.join(out_dir, name + ".c")
    so = os.path.join(out_dir, name + ".so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
                    "-fPIC", "-shared", "-w", "-o", so, c, "-lm"], check=True,
                   cwd=os.path.join(ROOT, "oracle"))
    return so


def _pins_pass(so):
    env = dict(os.environ, MOERO_LIB=so, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_oracle_pins.py"),
                        "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    return r.returncode == 0


def test_every_mutant_fails_a_pin():
    base = open(SRC).read()
    for name, old, new in MUTANTS:
        assert base.count(old) == 1, f"mutation site not unique/found: {name}"
    with tempfile.TemporaryDirectory() as tmp:
        # -I so the mutant finds moero.h
        base_inc = base.replace('#include "moero.h"', f'#include "{os.path.join(ROOT, "oracle", "moero.h")}"')
        jobs = [("original", base_inc)]
        for i, (name, old, new) in enumerate(MUTANTS):
            jobs.append((name, base_inc.replace(old, new)))
        sos = [(name, _build(text, tmp, f"m{i}")) for i, (name, text) in enumerate(jobs)]
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 2)) as ex:
            results = list(ex.map(lambda ns: (ns[0], _pins_pass(ns[1])), sos))
    assert results[0] == ("original", True), "the unmutated oracle must pass its pins"
    survivors = [name for name, passed in results[1:] if passed]
    assert not survivors, f"mutants no pin catches: {survivors}"
