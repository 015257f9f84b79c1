"""Builds libfa.so (the HIP kernels and the C ABI of include/fa.h) for gfx950 with hipcc.

``python -m flashattention_forward_flash_amd.build`` or ``build()``; the library lands
in-tree next to this file so that it travels with the source tree.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "fa_fwd.hip")
LIB = os.path.join(HERE, "libfa.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-shared",
    # every fused multiply-add is explicit in the source: identical bits on every code path
    "-ffp-contract=off",
    # no packed-fp32 VALU instructions (v_pk_{add,mul,fma}_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose=False, extra=()):
    cmd = [HIPCC, *FLAGS, *extra, SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    out = "\n".join(l for l in (res.stdout + res.stderr).splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{out}")
    os.replace(LIB + ".tmp", LIB)
    if verbose and out.strip():
        print(out)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
    print(LIB)
