"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer runs
the whole pin suite cleanly (CPU only).

oracle/moero.c is compiled with -fsanitize=address,undefined (every report
fatal), and tests/test_oracle_pins.py runs in a child process against that
build (MOERO_LIB), with the sanitizer runtime preloaded so the Python
interpreter can load an instrumented library. Any out-of-bounds access,
use-after-free, signed overflow, misaligned access or other undefined
behaviour in the oracle on the pins' inputs fails the test with the
sanitizer's report.
"""
import os
import subprocess
import sys
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "moero.c")


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _run_pins_sanitized(src_text, tmp):
    asan = _runtime("libasan.so")
    ubsan = _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc's sanitizer runtimes are not installed")
    c = os.path.join(tmp, "moero_san.c")
    so = os.path.join(tmp, "libmoero_san.so")
    with open(c, "w") as f:
        f.write(src_text.replace('#include "moero.h"',
                                 f'#include "{os.path.join(ROOT, "oracle", "moero.h")}"'))
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off",
                    "-fno-fast-math", "-fPIC", "-shared", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-o", so, c, "-lm"], check=True)
    # reports go to files (the child pytest's own capture would swallow them
    # when the sanitizer ends the process)
    log = os.path.join(tmp, "san")
    env = dict(os.environ, MOERO_LIB=so, OMP_NUM_THREADS="2",
               LD_PRELOAD=f"{asan}:{ubsan}",
               ASAN_OPTIONS=f"detect_leaks=0:abort_on_error=0:halt_on_error=1:log_path={log}",
               UBSAN_OPTIONS=f"halt_on_error=1:print_stacktrace=1:log_path={log}")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_oracle_pins.py"),
                        "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    reports = "".join(open(os.path.join(tmp, f)).read() for f in sorted(os.listdir(tmp))
                      if f.startswith("san"))
    return r.returncode, r.stdout + r.stderr + reports


def test_pin_suite_under_address_and_undefined_behaviour_sanitizers():
    with tempfile.TemporaryDirectory() as tmp:
        rc, out = _run_pins_sanitized(open(SRC).read(), tmp)
    assert rc == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]


def test_sanitized_build_reports_a_planted_overflow():
    # the harness itself: a copy of the oracle that writes one element past
    # a heap array must be stopped by AddressSanitizer
    src = open(SRC).read()
    old = "for (int32_t e = 0; e < N; ++e) mean[e] /= (double)T;"
    assert src.count(old) == 1
    with tempfile.TemporaryDirectory() as tmp:
        rc, out = _run_pins_sanitized(src.replace(old, old.replace("e < N", "e <= N")), tmp)
    assert rc != 0 and "heap-buffer-overflow" in out, out[-2000:]
