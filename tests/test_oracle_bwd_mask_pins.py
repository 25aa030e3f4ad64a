"""The masked gradient oracle against torch autograd, finite differences, the
unmasked and causal gradient oracle, closed forms and invariants (see
oracle_bwd_mask_pins.py)."""
import pytest

import oracle
from oracle_bwd_mask_pins import BWD_MASK_PINS


@pytest.fixture(scope="module")
def lib():
    oracle.build()
    return oracle.LIB_PATH


@pytest.mark.parametrize("pin", BWD_MASK_PINS, ids=[p.__name__ for p in BWD_MASK_PINS])
def test_oracle_bwd_mask_pin(lib, pin):
    pin(lib)
