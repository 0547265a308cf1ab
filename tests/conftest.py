"""Shared pytest configuration.

Markers: ``gpu`` marks tests that need an MI355X (gfx950) device; the CPU suite
runs with ``-m "not gpu"``.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU (runs on the GPU box)")


def golden(name: str) -> dict:
    """Parse tests/golden/<name>: 'key = value' lines; '#' starts a comment."""
    out = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            k, v = (s.strip() for s in line.split("=", 1))
            out[k] = v
    return out


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle._load()
    return oracle
