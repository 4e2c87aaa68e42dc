"""The CPU oracle against its pins (see tests/oracle_pins.py)."""
import pytest


import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.default())
