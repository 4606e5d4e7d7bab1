"""The oracle against the hand-derived worked example under tests/golden/
(exact fractions; the fixture cites the passages it follows and shows its
derivation), and that this example catches every oracle mutant by itself."""

import shutil
import subprocess

import pytest

import oracle
from tests import pins


def test_oracle_reproduces_the_worked_example():
    pins.pin_worked_example(oracle)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_the_worked_example_alone_catches_every_mutant(tmp_path):
    """Every mutant of the recurrence's arithmetic, the output scale included (the
    example also runs at scale 1/2), changes the example's numbers."""
    import os
    from tests.test_oracle import MUTANTS
    src = open(os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")).read()
    missed = []
    for name, (old, new) in sorted(MUTANTS.items()):
        path = tmp_path / f"{name}.c"
        path.write_text(src.replace(old, new))
        lib = str(tmp_path / f"lib{name}.so")
        subprocess.check_call(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", lib, str(path), "-lm"])
        try:
            pins.pin_worked_example(oracle.load_variant(lib))
            missed.append(name)
        except AssertionError:
            pass
    assert missed == [], missed
