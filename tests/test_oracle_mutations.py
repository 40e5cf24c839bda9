"""Every planted mistake in the oracle is caught by the oracle's pins.

tests/oracle_mutants.py lists plausible slips (a dropped term, a wrong sign,
a wrong operand or index, a wrong tie or split rule).  For each, the pin tests
of the oracle run in a fresh process with the mutant loaded in place of the
oracle module, and at least one of them must fail.  A mutant that survives
names a gap in the pins.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

from tests.oracle_mutants import DIAG, MUTANTS, ROOT

PINS = ["tests/test_oracle_dense.py", "tests/test_oracle_select.py", "tests/test_oracle_sparse.py",
        "tests/test_oracle_pddp.py", "tests/test_oracle_diagnostics.py"]


def _run(name: str) -> tuple[str, int, str]:
    files = ["tests/test_oracle_diagnostics.py"] if MUTANTS[name][0] == DIAG else PINS
    env = dict(os.environ, MCS_ORACLE_MUTANT=name, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", *files, "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    return name, r.returncode, r.stdout[-1500:] + r.stderr[-500:]


def test_every_planted_mistake_fails_a_pin():
    with ThreadPoolExecutor(max_workers=4) as pool:
        results = list(pool.map(_run, sorted(MUTANTS)))
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    broken = [(n, rc, out) for n, rc, out in results if rc not in (0, 1)]
    assert not broken, f"mutants that did not run as tests: {[(n, rc) for n, rc, _ in broken]}\n{broken[0][2]}"
    assert not survivors, f"mutants no pin catches: {[n for n, _ in survivors]}"
