import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU-side check")
    # the sanitized runs of tests/test_sanitizers.py: route the binding and the
    # oracle to their ASan + UBSan builds for the whole session
    if os.environ.get("SWR_SANITIZED_LIB"):
        import sliding_window_ring_amd as swr

        swr.lib = swr._load(os.environ["SWR_SANITIZED_LIB"])
    if os.environ.get("ORACLE_SANITIZED_LIB"):
        import ctypes

        import oracle

        oracle._lib = oracle._bind(ctypes.CDLL(os.environ["ORACLE_SANITIZED_LIB"]))


@pytest.fixture(scope="session")
def orc():
    import oracle

    oracle.build()
    return oracle
