"""The fp64 oracle checked against what the pages and mathematics fix
(closed forms, reductions, invariants, brute force); see oracle_pins.py."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin, lib):
    pin(lib)
