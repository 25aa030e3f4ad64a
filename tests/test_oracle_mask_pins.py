"""The general-mask oracle against the plain oracle on slices and closed forms
(see oracle_mask_pins.py)."""
import pytest

import oracle
from oracle_mask_pins import MASK_PINS


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.LIB_PATH


@pytest.mark.parametrize("pin", MASK_PINS, ids=[p.__name__ for p in MASK_PINS])
def test_oracle_mask_pin(lib, pin):
    pin(lib)
