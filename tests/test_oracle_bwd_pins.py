"""The gradient oracle against finite differences of the forward oracle, a
library routine, closed forms and invariants (see oracle_bwd_pins.py)."""
import pytest

import oracle
from oracle_bwd_pins import BWD_PINS


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.LIB_PATH


@pytest.mark.parametrize("pin", BWD_PINS, ids=[p.__name__ for p in BWD_PINS])
def test_oracle_bwd_pin(lib, pin):
    pin(lib)
