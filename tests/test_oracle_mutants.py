"""The oracle's CPU pins catch plausible mistakes planted in the oracle.

Each mutant of tests/oracle_mutants.py (a wrong table entry, constant,
offset, rounding tie, sign, index, operand order, normalisation or missing
transpose, one at a time) is loaded in a fresh pytest process through the
FP4_ORACLE_MUTATION hook of conftest.py, and the oracle pin tests
(tests/test_oracle_*.py) must fail on it.  CPU only; nothing here touches
the HIP library."""
import json
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from oracle_mutants import MUTANTS

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _pin_files():
    return sorted(os.path.join(HERE, f) for f in os.listdir(HERE)
                  if f.startswith("test_oracle_") and f.endswith(".py") and f != os.path.basename(__file__))


def _run(mutant):
    name, mod, old, new = mutant
    env = dict(os.environ, FP4_ORACLE_MUTATION=json.dumps([mod, old, new]),
               OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1")
    p = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *_pin_files()],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, p.returncode, p.stdout[-600:]


def test_every_planted_mistake_fails_a_pin():
    with ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        results = list(ex.map(_run, MUTANTS))
    survived = [n for n, rc, _ in results if rc == 0]
    broken = [(n, rc, out) for n, rc, out in results if rc not in (0, 1)]
    assert not broken, f"mutants that did not run as test failures: {broken}"
    assert not survived, f"mistakes no pin catches: {survived}"
