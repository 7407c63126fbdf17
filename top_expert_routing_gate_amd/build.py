"""Build libmoer.so (the router's C-ABI library) for gfx950 with hipcc.

Sources are compiled in parallel into ``_build/`` at the repo root and linked
into ``top_expert_routing_gate_amd/libmoer.so`` (kept in-tree so that the
built library travels with the source tree).
"""
import concurrent.futures
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmoer.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["moer_api.hip", "gate_gemm.hip", "route_rows.hip", "route_small.hip", "route_fused.hip", "score_topk.hip", "layout.hip",
           "stats.hip", "dispatch_combine.hip",
           "forcible.hip", "capacity.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"  # host pass warns about the device-only feature
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msg}")
    return obj, msg


def build_library(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    if verbose:
        for obj, msg in results:
            if msg.strip():
                print(msg)
    objs = [o for o, _ in results]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_library(verbose=True))
