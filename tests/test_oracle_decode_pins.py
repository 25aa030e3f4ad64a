"""The decode oracle against the plain oracle and closed forms (see
oracle_decode_pins.py)."""
import pytest

import oracle
from oracle_decode_pins import DECODE_PINS


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.LIB_PATH


@pytest.mark.parametrize("pin", DECODE_PINS, ids=[p.__name__ for p in DECODE_PINS])
def test_oracle_decode_pin(lib, pin):
    pin(lib)
