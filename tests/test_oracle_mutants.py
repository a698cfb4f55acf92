"""Every planted mistake in the oracle fails at least one of its pins.

For each mutant of tests/oracle_mutants.py the oracle's pin suites run in a
subprocess with the mistake planted (LQ_ORACLE_MUTANT), and must fail; the
same suites without a mutant pass in the main run.  This shows that the
pins tie the oracle to the pages and the mathematics closely enough that a
plausible slip anywhere in it is caught.  CPU only.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from tests import oracle_mutants

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_SUITES = ["tests/test_oracle_pins.py", "tests/test_oracle_dense_comp.py"]


def _run(name):
    env = dict(os.environ, LQ_ORACLE_MUTANT=name, PYTHONDONTWRITEBYTECODE="1")
    env.pop("PYTEST_XDIST_WORKER", None)
    cmd = [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-p", "no:xdist",
           "-m", "not gpu", *PIN_SUITES]
    res = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, res.returncode, res.stdout[-2000:] + res.stderr[-2000:]


@pytest.fixture(scope="module")
def mutant_runs():
    with ThreadPoolExecutor(max_workers=4) as ex:
        return {name: (rc, out) for name, rc, out in ex.map(_run, sorted(oracle_mutants.MUTANTS))}


@pytest.mark.parametrize("name", sorted(oracle_mutants.MUTANTS))
def test_planted_mistake_fails_a_pin(name, mutant_runs):
    rc, out = mutant_runs[name]
    # pytest exit code 1: tests ran and at least one failed (2-5 would be an
    # error of the harness itself, not a caught mistake)
    assert rc == 1, f"mutant {name}: pin suites exited {rc}\n{out}"
    assert "failed" in out, out
