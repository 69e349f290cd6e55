import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_terminal_summary(terminalreporter):
    """Worst ratio of a GEMM's error to its element-wise bound, per test."""
    try:
        from gemm_check import WORST
    except ImportError:
        return
    if WORST:
        terminalreporter.write_line("GEMM |dY| / (4 K 2^-24 sum|a w|), worst per test:")
        for name, r in sorted(WORST.items()):
            terminalreporter.write_line(f"  {name}: {r:.3e}")
