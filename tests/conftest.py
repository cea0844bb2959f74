"""Shared pytest set-up: the repository root on sys.path and the ``gpu`` marker.

Tests marked ``gpu`` call the HIP library through its C ABI and need a gfx950
device; everything else runs on the CPU only.
"""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
