import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest


class _HostOnly:
    """A host-only build of the validation and planning code (WQ_HOST_LIBRARY, the
    sanitizer build): a test that calls anything else is skipped."""

    def __init__(self, L):
        self._L = L

    def __getattr__(self, name):
        if not hasattr(self._L, name):
            pytest.skip(f"{name} is not in the host-only library")
        return getattr(self._L, name)


@pytest.fixture(scope="session")
def wqlib():
    """The C-ABI library, built in-tree first if it is missing (CPU-side cross-compile);
    or, when WQ_HOST_LIBRARY names one, a host-only build of its validation and planning
    code."""
    import ctypes
    import weight_quantized_gemm_amd as W
    host = os.environ.get("WQ_HOST_LIBRARY")
    if host:
        return _HostOnly(W.declare(ctypes.CDLL(host)))
    if not os.path.exists(W.library_path):
        from weight_quantized_gemm_amd import build
        build.build(verbose=False)
    return W.lib()
