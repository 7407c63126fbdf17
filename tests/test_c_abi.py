"""The plain-C driver of the router's C ABI, on the host (no GPU): it is
built, links the in-tree libmoer.so, and rejects bad arguments and a bad
input file before it touches the device."""
import os
import struct
import subprocess

import pytest

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "moer_route_c")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def exe():
    if not os.path.exists(EXE):
        pytest.skip("the C driver is not built (run __graft_entry__.build())")
    return EXE


def test_links_the_in_tree_library(exe):
    r = subprocess.run(["ldd", exe], capture_output=True, text=True, timeout=60)
    lib = os.path.join(ROOT, "top_expert_routing_gate_amd", "libmoer.so")
    line = next(l for l in r.stdout.splitlines() if "libmoer.so" in l)
    assert os.path.realpath(line.split("=>")[1].split("(")[0].strip()) == os.path.realpath(lib)


def test_usage_and_bad_inputs(exe, tmp_path):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "usage" in r.stderr
    r = subprocess.run([exe, str(tmp_path / "missing.bin"), str(tmp_path / "o.bin")],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "cannot open" in r.stderr
    bad = tmp_path / "bad.bin"
    bad.write_bytes(struct.pack("<12i", 0x1234, 1, 64, 128, 4, 1, 1, 1, 0, 0, 1, 0) +
                    struct.pack("<f", 1e-3))
    r = subprocess.run([exe, str(bad), str(tmp_path / "o.bin")], capture_output=True, text=True,
                       timeout=60)
    assert r.returncode == 1 and "bad input header" in r.stderr
    short = tmp_path / "short.bin"
    short.write_bytes(struct.pack("<12i", 0x524F454D, 1, 64, 128, 4, 1, 1, 1, 0, 0, 1, 0) +
                      struct.pack("<f", 1e-3) + b"\0" * 100)
    r = subprocess.run([exe, str(short), str(tmp_path / "o.bin")], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 1 and "short input file" in r.stderr
