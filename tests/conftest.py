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


@pytest.fixture(scope="session")
def q4():
    """The HIP library binding; GPU tests fail (not skip) without a GPU or
    without the built library."""
    import torch
    assert torch.cuda.is_available(), "gpu tests need a visible MI355X"
    import int4_quantized_decode_q4_amd as q4mod
    return q4mod


def pytest_runtest_setup(item):
    # name the case before any GPU work, so a fault still leaves a trace
    if item.get_closest_marker("gpu") is not None:
        print(f"\n[gpu-case] {item.nodeid}", flush=True)
