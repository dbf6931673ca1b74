"""Each planted slip in a copy of the oracle must make the pin suite fail."""

import os
import subprocess
import sys

import pytest

from tests_mutants import MUTANTS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("idx", range(len(MUTANTS)), ids=[m[0] for m in MUTANTS])
def test_pins_detect_mutant(idx):
    env = dict(os.environ, ORACLE_MUTANT=str(idx), OPENBLAS_NUM_THREADS="1", OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert "mutant %d no longer applies" % idx not in r.stdout + r.stderr
    assert r.returncode == 1, "pins did not catch mutant %r:\n%s" % (MUTANTS[idx][0], r.stdout[-2000:])
