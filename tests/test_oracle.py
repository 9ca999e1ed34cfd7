"""The float64 oracle against its pins (CPU only)."""

import pytest

import oracle
from tests import pins


@pytest.mark.parametrize("pin", pins.PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle)
