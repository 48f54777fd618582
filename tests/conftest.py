"""Shared pytest configuration.

Markers:
  gpu  -- needs a real MI355X (gfx950); everything else runs on the CPU.

Tests that need a compiled library build it once if it is missing (the oracle
with gcc, libqmm with hipcc), so a fresh checkout can run ``pytest -m "not gpu"``.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X GPU (gfx950)")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle


@pytest.fixture(scope="session")
def qmm_lib():
    """libqmm.so, built in-tree with hipcc if it is not there yet."""
    from quantized_matmul_ggml_amd import binding, build
    if not os.path.exists(binding.LIB_PATH):
        build.build()
    return binding
