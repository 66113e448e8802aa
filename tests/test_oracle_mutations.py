"""The oracle's pins catch plausible mistakes: each mutant in oracle_mutants.py (a slip
planted in one oracle function, on the CPU) must make tests/test_oracle_pins.py fail,
and the unmutated oracle must pass them.  Each run is a pytest subprocess with the
mutant plugin loaded, so no mutant leaks into this process."""
import os
import subprocess
import sys

import pytest

from oracle_mutants import MUTANTS

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _run_pins(mutant: str) -> subprocess.CompletedProcess:
    env = dict(os.environ)
    env["DJV_ORACLE_MUTANT"] = mutant
    env["PYTHONPATH"] = os.pathsep.join([HERE, ROOT, env.get("PYTHONPATH", "")])
    cmd = [sys.executable, "-m", "pytest", os.path.join(HERE, "test_oracle_pins.py"), "-x", "-q",
           "-p", "oracle_mutants", "-p", "no:cacheprovider", "-m", "not gpu"]
    return subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


def test_pins_pass_without_mutant():
    r = _run_pins("")
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-2000:]


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_pins_catch_mutant(mutant):
    r = _run_pins(mutant)
    # exit code 1: tests ran and at least one failed (not an import or usage error)
    assert r.returncode == 1, f"{mutant} was not caught:\n{r.stdout[-2000:]}{r.stderr[-2000:]}"
