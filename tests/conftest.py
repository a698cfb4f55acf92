import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running check")


def pytest_sessionstart(session):
    # a planted oracle mistake, set only by tests/test_oracle_mutants.py in
    # the subprocesses it starts
    name = os.environ.get("LQ_ORACLE_MUTANT")
    if name:
        from tests import oracle_mutants
        oracle_mutants.apply(name)
