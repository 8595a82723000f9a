"""The oracle's pins catch planted mistakes (CPU only).

Each mutant in ``tests/_mutant.py`` plants one plausible mistake into the
oracle (a wrong GQA index, a missing transpose, a dropped scale, a wrong
merge weight, a wrong bf16 widening, a missing copy-on-write decrement, a
LIFO free pool, an off-by-one slot, a causal limit off by one, a window off
by one, E4M3 ties to odd, ...).  The test files named with it then run in a
fresh process against the planted mistake, and at least one of their tests
must fail (pytest exit status 1; an error while planting is status 3 and
fails this test).  A pin that lets a plausible mistake through is no pin.
"""
import concurrent.futures as cf
import os
import re
import subprocess
import sys

import pytest

from _mutant import MUTANTS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(name: str):
    files = MUTANTS[name][3]
    path = os.pathsep.join([ROOT, os.path.join(ROOT, "tests"), os.environ.get("PYTHONPATH", "")])
    env = dict(os.environ, PA_ORACLE_MUTANT=name, PYTHONDONTWRITEBYTECODE="1", PYTHONPATH=path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "_mutant",
                        "-p", "no:cacheprovider", "-m", "not gpu", *files],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode, (r.stdout + r.stderr)[-2000:]


@pytest.fixture(scope="module")
def outcomes():
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        return {name: (rc, tail) for name, rc, tail in ex.map(_run, sorted(MUTANTS))}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(outcomes, name):
    rc, tail = outcomes[name]
    # status 1 with a "N failed" summary: the plugin loaded, planted the
    # mistake, and a pin failed (a plugin that cannot load also exits with 1)
    assert rc == 1 and re.search(r"\b\d+ failed\b", tail), \
        f"mutant {name}: pytest exit status {rc} (1 = a pin failed)\n{tail}"
