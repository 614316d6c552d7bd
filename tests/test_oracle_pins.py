"""CPU: the oracle against its pins (hand-worked fixtures, closed forms,
constructed-exact inputs, bounds, brute force, special cases)."""
import pytest

import oracle.ref as ora
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_oracle_pin(pin):
    pin(ora)
