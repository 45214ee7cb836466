"""Build the CPU oracle, liboracle.so (g++, fp32, -ffp-contract=off, OpenMP).
Test infrastructure: only tests, the smoke check and the benchmark's CPU
baseline load it."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def build():
    subprocess.run(["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC",
                    "-shared", "-Wall", "-Wextra", "oracle.cpp", "-o", "liboracle.so.tmp"],
                   check=True, cwd=HERE)
    os.replace(os.path.join(HERE, "liboracle.so.tmp"), os.path.join(HERE, "liboracle.so"))


if __name__ == "__main__":
    build()
