"""The fp64 oracle against brute force, torch's SDPA, closed forms and the
pages' printed tables (see tests/oracle_pins.py)."""
import pytest

import oracle.attention as A
from tests.oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin(A)
