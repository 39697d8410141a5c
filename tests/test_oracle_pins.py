"""The oracle against its pins (hand-worked values, brute force, closed forms, invariants)."""
import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.get())
