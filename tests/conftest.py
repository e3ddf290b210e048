import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle():
    from oracle import oracle as O

    O.lib()
    return O


# Full-size decode inputs (seeded; generated once per session, on first use).
@pytest.fixture(scope="session")
def decode_full():
    from workloads import decode_inputs

    return decode_inputs("decode")


@pytest.fixture(scope="session")
def truncated_full():
    from workloads import decode_inputs

    return decode_inputs("truncated")
