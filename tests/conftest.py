import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (runs the HIP kernels)")


@pytest.fixture(scope="session")
def fa_lib():
    """libfa.so loaded through the binding (built first only if absent).

    FA_HOST_CAPI_LIB names another build of the C ABI to bind instead: the
    host-only sanitizer build of tests/test_host_sanitizers.py, for the host
    validation tests (it launches nothing)."""
    import exact_attention_12_amd as fa
    alt = os.environ.get("FA_HOST_CAPI_LIB")
    if alt:
        import ctypes
        fa._LIB = fa._bind(ctypes.CDLL(alt))
        return fa._LIB
    if not os.path.exists(fa.lib_path()):
        from exact_attention_12_amd import build
        build.build()
    return fa.load_library()


@pytest.fixture(scope="session")
def gpu():
    """The HIP device; a GPU test without one fails loudly instead of skipping."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    return torch.device("cuda:0")
