"""Build libsmoe.so, the MI355X (gfx950) routed-MoE layer library, in-tree."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["api.cpp", "router.hip", "ffn.hip", "ffn_gemv.hip", "ffn_mfma.hip", "norm.hip",
           "attn.hip", "noalloc.hip", "diag.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
         "-fvisibility=hidden", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
LIB = os.path.join(HERE, "libsmoe.so")


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = ["hipcc", *FLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True, cwd=CSRC)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
