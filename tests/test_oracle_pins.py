"""The oracle against its pins (see tests/pins_oracle.py)."""
import pytest

from pins_oracle import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(pin):
    pin()
