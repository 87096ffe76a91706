"""The fp64 oracle against its pins (CPU only)."""

import pytest

import oracle
import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)
