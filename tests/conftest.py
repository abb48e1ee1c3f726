import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    # Load (or compile) the oracle before any test touches the GPU: a compiler
    # started from a process that has initialised the GPU would be a program
    # started after GPU initialisation.
    import oracle
    oracle.default()
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle.default()
