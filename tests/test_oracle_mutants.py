"""The oracle's pins catch plausible mistakes planted in the oracle (CPU only).

For every mutant of ``tests/oracle_mutants.py`` the pin files run in a child
pytest process with that mistake planted in memory; at least one pin must
fail.  A control run with no mutant must pass.  A mutant that survived would
mean the oracle could carry that mistake unnoticed.
"""
import os
import subprocess
import sys

import pytest

from oracle_mutants import ENV, MUTANTS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = ["tests/test_oracle_pins.py", "tests/test_oracle_pins_next.py",
             "tests/test_oracle_mx_pins.py"]


def _run_pins(mutant):
    env = dict(os.environ)
    env.pop(ENV, None)
    if mutant:
        env[ENV] = mutant
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-rf", "-m", "not gpu",
                        "-p", "no:cacheprovider", *PIN_FILES],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    failed = [l for l in r.stdout.splitlines() if l.startswith("FAILED")]
    return r.returncode, failed, r.stdout[-2000:] + r.stderr[-2000:]


def test_pins_pass_without_mutant():
    rc, failed, tail = _run_pins(None)
    assert rc == 0, tail


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name):
    rc, failed, tail = _run_pins(name)
    assert rc == 1 and failed, f"mutant {name} survived the pins:\n{tail}"
    print(f"{name}: caught by {failed[0]}")
