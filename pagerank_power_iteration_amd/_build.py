"""Build libpr.so (the HIP library behind include/pr.h) in place with hipcc
for gfx950."""
from __future__ import annotations

import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libpr.so")
ARCH = os.environ.get("PR_OFFLOAD_ARCH", "gfx950")


def sources():
    return sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))


def hipcc_command(out: str) -> list[str]:
    return [
        "hipcc", "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-shared",
        "-Wall", "-Wno-unused-function",
        # never emit packed-fp32 arithmetic (v_pk_*_f32)
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"), "-I", os.path.join(PKG, "csrc"),
        "-o", out, *sources(),
    ]


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = hipcc_command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
