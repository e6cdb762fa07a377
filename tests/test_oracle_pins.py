"""The oracle against its pins (CPU only)."""
import os
import subprocess

import pytest

import oracle as oracle_pkg
from tests.oracle_pins import PINS


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(oracle, pin):
    assert oracle.mutant == 0
    pin(oracle)


# Planted mistakes, one per build (see ORACLE_MUTANT in oracle/moe_oracle.c):
# 1 drops the W3 factor, 2 flips silu's sign, 3 selects the smallest logits,
# 4 normalises over all experts, 5 transposes W_g, 6 transposes W2,
# 7 swaps the slot weights in the combine, 8 reverses the permute order,
# 9 takes the 1st-2nd instead of the 2nd-3rd margin.
MUTANTS = list(range(1, 16))


@pytest.mark.parametrize("mutant", MUTANTS)
def test_pins_catch_planted_mistake(tmp_path, mutant):
    path = str(tmp_path / f"liboracle_m{mutant}.so")
    try:
        oracle_pkg.build(path, mutant=mutant)
    except (OSError, subprocess.CalledProcessError) as exc:  # pragma: no cover
        pytest.skip(f"gcc unavailable: {exc}")
    o = oracle_pkg.Oracle(path)
    assert o.mutant == mutant
    caught = []
    for pin in PINS:
        try:
            pin(o)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {mutant} passes every pin"
