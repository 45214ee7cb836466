"""Build liboracle_asan.so: the CPU oracle with AddressSanitizer and
UndefinedBehaviorSanitizer (g++, host code only), for running the oracle's
pins under the sanitizers (tests/test_sanitizers.py).  Load it by setting
ORACLE_LIBRARY to its path and preloading g++'s libasan."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle_asan.so")


def build() -> str:
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-ffp-contract=off", "-fopenmp", "-fPIC",
                    "-shared", "-Wall", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "oracle.cpp", "-o", LIB + ".tmp"],
                   check=True, cwd=HERE)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def runtime() -> str:
    """The sanitizer runtime to preload into an uninstrumented python."""
    return subprocess.run(["g++", "-print-file-name=libasan.so"], check=True,
                          capture_output=True, text=True).stdout.strip()


if __name__ == "__main__":
    print(build())
