"""The CPU oracle against the pages' printed examples, closed forms, a library
routine and invariants of the definition (see oracle_pins.py)."""
import pytest

import oracle
from oracle_pins import PINS


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.LIB_PATH


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(lib, pin):
    pin(lib)
