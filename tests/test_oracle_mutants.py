"""The oracle's pins catch plausible mistakes: each mutant in
tests/oracle_mutants.py plants one mistake in the oracle (CPU only), and the pin
suite, run under it in a fresh process, must fail."""
import os
import subprocess
import sys

import pytest

from oracle_mutants import MUTANTS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    env = dict(os.environ, ORACLE_MUTANT=name)
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-q", "-x", "-p",
                        "no:cacheprovider", "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=900)
    assert r.returncode == 1 and " failed" in r.stdout, (
        f"the pins did not catch mutant {name} (exit {r.returncode}):\n{r.stdout[-2000:]}\n{r.stderr[-2000:]}")
