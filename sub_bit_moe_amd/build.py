"""Build libsbm.so in-tree with hipcc for gfx950.

Usage: python -m sub_bit_moe_amd.build   (or __graft_entry__.build()).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libsbm.so")

SOURCES = ["sbm_host.cpp", "sbm_gpu.hip", "sbm_gen.hip", "sbm_dense.hip"]
ARCH = os.environ.get("SBM_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsbm)")


def command(out: str) -> list:
    return [
        hipcc(), "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
        # packed fp32 VALU forms are disabled for all device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-ffp-contract=off", "-Wall", "-Wno-unused-result",
        f"-I{INCLUDE}", f"-I{CSRC}",
        *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out,
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("building libsbm.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
