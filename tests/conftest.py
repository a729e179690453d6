import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# tests/test_oracle_mutants.py runs the pin suite with one planted oracle mistake
if os.environ.get("ORACLE_MUTANT"):
    import oracle_mutants

    oracle_mutants.apply(os.environ["ORACLE_MUTANT"])


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity cases (seconds to a minute each)")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")
