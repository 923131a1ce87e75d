"""Every planted oracle mistake (tests/oracle_mutations.py) fails at least
one pin of tests/test_oracle_pins.py that is not a comparison with the
pure-Python twin: the pins tie the oracle to worked examples, closed forms,
invariants and other people's code, not only to a second copy of the same
formulas.  Each mutation runs the pins in a process of its own (CPU only)."""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle_mutations import MUTATIONS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# the twin comparisons restate the oracle's formulas: a mutation must be
# caught without them
NOT_TWIN = "not twin and not size_one_is_identity"


def _run_pins(name):
    env = dict(os.environ, ORACLE_MUTATION=name)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "-k", NOT_TWIN, os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    return name, r.returncode, r.stdout


@pytest.fixture(scope="module")
def outcomes():
    with ThreadPoolExecutor(max_workers=4) as ex:
        return {name: (rc, out) for name, rc, out in ex.map(_run_pins, sorted(MUTATIONS))}


def test_unmutated_pins_pass_without_the_twin():
    name, rc, out = _run_pins("")
    assert rc == 0, out[-2000:]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(outcomes, name):
    rc, out = outcomes[name]
    # exit status 1: tests ran and at least one failed (2-5: usage or collection errors)
    assert rc == 1 and " failed" in out, f"mutation {name} not caught (exit {rc}):\n{out[-2000:]}"
