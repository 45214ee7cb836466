import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _ensure_built():
    """Build the CPU-side libraries only when nothing is built yet."""
    if not os.path.exists(os.path.join(ROOT, "synth", "libsynth.so")):
        from synth import build as sb
        sb.build_cpu()
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        from oracle import build as ob
        ob.build()


_ensure_built()
