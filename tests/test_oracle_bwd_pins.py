"""The fp64 backward oracle against finite differences, torch autograd,
closed forms and the full-sequence gradient (see tests/oracle_bwd_pins.py)."""
import pytest

import oracle.attention as A
import oracle.backward as G
from tests.oracle_bwd_pins import ALL_BWD_PINS


@pytest.mark.parametrize("pin", ALL_BWD_PINS, ids=[p.__name__ for p in ALL_BWD_PINS])
def test_bwd_pin(pin):
    pin(A, G)
