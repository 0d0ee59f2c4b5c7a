"""The oracle's pins catch plausible mistakes in it. For every planted mistake of
tests/_oracle_mutants.py (a dropped norm or residual, a wrong sign, index, offset, constant or
tie rule, swapped operands, in the elementary steps, the page model, the context append, the
block forward, the FP8 codes and the DSpark and DFlash2 heads), the pins in
tests/test_oracle_pins.py run in a child pytest process with that one mistake put in place of
the original function in memory; at least one pin must fail there (an ordinary test failure,
not a collection or plugin error). The oracle's file is never changed."""
import concurrent.futures as cf
import os
import subprocess
import sys

import _oracle_mutants as M

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _run(name):
    env = dict(os.environ, DFLASH_ORACLE_MUTANT=name,
               PYTHONPATH=HERE + os.pathsep + os.environ.get("PYTHONPATH", ""))
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(HERE, "test_oracle_pins.py"), "-x", "-q",
                        "-p", "_oracle_mutants", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return name, r.returncode, (r.stdout + r.stderr)[-2000:]


def test_every_planted_mistake_fails_a_pin():
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(_run, sorted(M.MUTANTS)))
    survived = [n for n, rc, _ in results if rc == 0]
    broken = [(n, rc, out) for n, rc, out in results if rc not in (0, 1)]
    assert not broken, "mutant runs that did not reach the pins: " + "; ".join(
        f"{n} (exit {rc}): {out[-300:]}" for n, rc, out in broken)
    assert not survived, f"planted mistakes no pin catches: {survived}"
