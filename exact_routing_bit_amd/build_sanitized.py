"""Build libsmoe_asan.so: libsmoe with AddressSanitizer and
UndefinedBehaviorSanitizer on its host code (argument validation and
launch set-up; the gfx950 device code is built as usual), for running the
C-ABI tests under the sanitizers on the host (tests/test_sanitizers.py).
Load it by setting SMOE_LIBRARY to its path and preloading clang's ASan
runtime (runtime())."""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsmoe_asan.so")


def build() -> str:
    import importlib.util
    spec = importlib.util.spec_from_file_location("_smoe_build", os.path.join(HERE, "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    host_only = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-g"]
    subprocess.run(["hipcc", *b.FLAGS, *host_only, *b.SOURCES, "-o", LIB + ".tmp"], check=True,
                   cwd=CSRC)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def runtime() -> str:
    """clang's ASan runtime (with its UBSan handlers) to preload into python."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise FileNotFoundError("clang's libclang_rt.asan-x86_64.so")
    return hits[-1]


if __name__ == "__main__":
    print(build())
