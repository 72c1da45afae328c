"""pytest setup: the repository root on sys.path and the ``gpu`` marker.

Tests marked ``gpu`` need an MI355X (gfx950) and call the HIP library through
its C ABI; everything else runs on a CPU-only machine.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an AMD gfx950 GPU and the built HIP library")
