"""Build tests/c_abi/moer_route_c, the plain-C driver of the router's C ABI.

It is compiled with the host C compiler (gcc, C11) against include/moer.h and
the HIP runtime's C API, and linked with the in-tree libmoer.so (found at run
time through an $ORIGIN-relative rpath) and libamdhip64. The HIP headers
need the platform named when a plain C compiler includes them
(__HIP_PLATFORM_AMD__); hipcc would name it itself.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "moer_route_c.c")
EXE = os.path.join(HERE, "moer_route_c")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CC = os.environ.get("CC", "gcc")


def build_driver():
    pkg = os.path.join(ROOT, "top_expert_routing_gate_amd")
    tmp = EXE + ".tmp"
    cmd = [CC, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), SRC,
           "-o", tmp, "-L", pkg, "-lmoer", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../top_expert_routing_gate_amd",
           "-Wl,-rpath," + os.path.join(ROCM, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("building the C driver failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build_driver())
