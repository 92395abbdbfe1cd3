"""CPU: the oracle against its pins (see tests/pins.py for what each pins)."""
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle)
