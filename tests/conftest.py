import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# a planted oracle mistake (tests/oracle_mutations.py), only when the pins are
# run by tests/test_oracle_mutations.py to show that they catch it
if os.environ.get("ORACLE_MUTATION"):
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    import oracle_mutations

    oracle_mutations.apply(os.environ["ORACLE_MUTATION"])


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running GPU case at full workload size")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
