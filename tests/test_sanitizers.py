"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

The oracle (built with g++) and libsmoe's host code (argument validation and
launch set-up, built with hipcc, the sanitizers on the host side only) are
rebuilt with both sanitizers, and the oracle's pins and the C-ABI tests run
against those builds in child processes, each with its compiler's runtime
preloaded (python itself is not instrumented).  Any sanitizer report fails
the child and with it this test."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _load(path, name):
    import importlib.util
    spec = importlib.util.spec_from_file_location(name, path)
    m = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(m)
    return m


def _run(test_file, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", os.path.join(ROOT, "tests", test_file)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    return out


def test_oracle_pins_under_sanitizers():
    path = os.path.join(ROOT, "oracle", "build_sanitized.py")
    if not os.path.exists(path):
        pytest.skip("sanitizer build script not present")
    b = _load(path, "_oracle_asan_build")
    lib = b.build()
    out = _run("test_oracle.py", {"ORACLE_LIBRARY": lib, "LD_PRELOAD": b.runtime()})
    assert "passed" in out


def test_abi_validation_under_sanitizers():
    path = os.path.join(ROOT, "exact_routing_bit_amd", "build_sanitized.py")
    if not os.path.exists(path):
        pytest.skip("sanitizer build script not present")
    b = _load(path, "_smoe_asan_build")
    lib = b.build()
    out = _run("test_abi.py", {"SMOE_LIBRARY": lib, "LD_PRELOAD": b.runtime()})
    assert "passed" in out
