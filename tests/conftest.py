"""pytest configuration: the ``gpu`` marker and shared fixtures.

Tests marked ``gpu`` need an MI355X (gfx950) and the built HIP library; all
others run on the CPU.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.load()
