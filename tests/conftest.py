"""Shared pytest setup: the ``gpu`` marker, import paths and the built libraries.

``-m "not gpu"`` runs everywhere (oracle pins, host logic, library exports);
``-m gpu`` needs an MI355X and compares the HIP path with the CPU oracle.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; compares with the CPU oracle")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
