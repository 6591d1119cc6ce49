"""The fp64 oracle against its pins (CPU only)."""
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle)
