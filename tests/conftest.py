import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# The library replaces its configuration table with SKINNY_CONFIG when that is set (read once,
# on first use); the tests check the table, so a value left in the environment must not reach
# them. The override's own test sets it in child processes.
os.environ.pop("SKINNY_CONFIG", None)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    # GPU tests are marked explicitly; nothing else to do here.
    return None


@pytest.fixture(scope="session")
def oracle_lib():
    import oracle
    return oracle.default()
