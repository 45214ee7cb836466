"""Build the synthetic-input generators: libsynth.so (gcc, CPU) and
libsynth_gpu.so (hipcc, gfx950).  Both use -ffp-contract=off so that they
produce the same bits."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _run(cmd):
    subprocess.run(cmd, check=True, cwd=HERE)


def build_cpu():
    _run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
          "synth.c", "-o", "libsynth.so.tmp", "-lm"])
    os.replace(os.path.join(HERE, "libsynth.so.tmp"), os.path.join(HERE, "libsynth.so"))


def build_gpu():
    _run(["hipcc", *HIP_FLAGS, "synth_gpu.hip", "-o", "libsynth_gpu.so.tmp"])
    os.replace(os.path.join(HERE, "libsynth_gpu.so.tmp"), os.path.join(HERE, "libsynth_gpu.so"))


def build():
    build_cpu()
    build_gpu()


if __name__ == "__main__":
    build()
