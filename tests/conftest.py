"""Shared pytest setup.

Markers: ``gpu`` marks tests that launch HIP kernels and need an MI355X.
Everything else runs on a CPU-only host.
"""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (gfx950) to run HIP kernels")


@pytest.fixture(scope="session")
def mvs_lib():
    """The built HIP library, built once if no build is present."""
    from masked_varlen_softmax_amd import build as _build

    if not os.path.exists(_build.library_path()):
        _build.build_library()
    import masked_varlen_softmax_amd as mvs

    return mvs.lib()
