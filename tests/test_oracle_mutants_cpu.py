"""The oracle's pins must kill every planted mistake of the mutation sweep in
``tests/oracle_mutants.py``, except the mutants it lists as equivalent."""
import os
import shutil
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
import oracle_mutants  # noqa: E402


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc to build the mutants")
def test_pins_kill_every_non_equivalent_mutant():
    res = oracle_mutants.sweep(workers=min(8, os.cpu_count() or 1))
    survivors = sorted(nm for nm, (killed, _) in res.items() if not killed)
    assert survivors == sorted(oracle_mutants.EQUIVALENT), {nm: res[nm][1] for nm in survivors}
