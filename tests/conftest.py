import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long CPU test")


def pytest_sessionstart(session):
    # The oracle's matrices in these tests are small: one BLAS thread is faster than a pool
    # spinning over many cores (the oracle's generation check took 2.6 s single-threaded and
    # up to 48 s with 16 BLAS threads on a GPU host).
    try:
        from threadpoolctl import threadpool_limits
        session.config._zo_blas_limit = threadpool_limits(limits=1)
    except Exception:
        pass
