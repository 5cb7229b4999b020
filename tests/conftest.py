import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running parity case")


def golden_lines(name):
    """Non-comment, non-blank lines of a golden fixture file."""
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.lstrip().startswith("#")]
