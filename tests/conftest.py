import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, TESTS):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    src_m = os.path.getmtime(oracle.SOURCE)
    hdr_m = os.path.getmtime(os.path.join(os.path.dirname(oracle.SOURCE), "gdn_oracle.h"))
    if not os.path.exists(oracle.LIBRARY) or os.path.getmtime(oracle.LIBRARY) < max(src_m, hdr_m):
        oracle.build()
    return oracle.load()
