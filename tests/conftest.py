"""Shared pytest configuration: the ``gpu`` marker and small helpers."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def root_dir():
    return ROOT


def pytest_sessionstart(session):
    """On a host without a GPU, build libfos.so if it is missing so that the C ABI
    checks can load it (on a GPU host the in-tree build is used as shipped)."""
    lib = os.path.join(ROOT, "fp4_block_quantization_amd", "libfos.so")
    if not os.path.exists(lib) and not os.path.exists("/dev/kfd"):
        from fp4_block_quantization_amd.build import build
        build(verbose=False)
