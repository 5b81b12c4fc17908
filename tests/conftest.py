import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
GOLDEN = os.path.join(ROOT, "tests", "golden")

# GCACHE_ORACLE_LIB names another build of the oracle's sources (the
# sanitized build of test_oracle_sanitized.py) for every test in this run.
if os.environ.get("GCACHE_ORACLE_LIB"):
    import oracle
    oracle._lib = oracle.lib(os.environ["GCACHE_ORACLE_LIB"])


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD Instinct MI355X (gfx950) GPU")


def load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.lib()
    return oracle
