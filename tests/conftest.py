import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest


@pytest.fixture(scope="session")
def wqlib():
    """The C-ABI library, built in-tree first if it is missing (CPU-side cross-compile)."""
    import weight_quantized_gemm_amd as W
    if not os.path.exists(W.library_path):
        from weight_quantized_gemm_amd import build
        build.build(verbose=False)
    return W.lib()
